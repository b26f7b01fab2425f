// Packing of ternary weights and per-token int8 activation quantization.
//
// Packing: each weight takes 2 bits (bitnet.cpp CPU tutorial at m.qwbw.cn,
// §1.1; the 2-bit format is called I2_S in "BitNet 1 位 LLM 独立推理引擎",
// conversion paragraph).  Code = trit + 1; the 64-row-tiled byte layout is
// stated in bt.h.
//
// Quantization: activations become 8-bit integers ("BitNet-rs" page, section
// "技术实现细节"), one absmax scale per token; the rounding and scale
// formula (round half to even, x * (127 / a), clamp +-127, a >= 1e-5) are the
// readings stated in bt.h.
#include <string.h>

#include "bt_internal.h"

namespace bt {
namespace {

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// One thread per (row, 64-input chunk): reads 64 trits, writes one 16-byte
// chunk of the packed layout.  Thread index L = (row block * kc + chunk) * 64
// + row % 64 equals the chunk's position in the output, so stores coalesce.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ t,
                                                   int64_t n, int64_t k,
                                                   int64_t total,
                                                   uint8_t* __restrict__ packed,
                                                   int32_t* n_invalid) {
  const int64_t L = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t kc = k >> 6;
  int bad = 0;
  if (L < total) {
    const int64_t r64 = L & 63;
    const int64_t bc = L >> 6;
    const int64_t c = bc % kc;
    const int64_t row = (bc / kc) * 64 + r64;
    uint32_t word[4] = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};
    if (row < n) {
      const int4* src = reinterpret_cast<const int4*>(t + row * k + c * 64);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // 16 consecutive trits: inputs 64 c + 16 w + 4 j + i (j, i < 4)
        const int4 v = src[w];
        const int32_t d4[4] = {v.x, v.y, v.z, v.w};
        uint32_t out = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int trit = (int8_t)((uint32_t)d4[j] >> (8 * i));
            uint32_t code = (uint32_t)(trit + 1);
            if (code > 2u) {
              code = 3u;
              ++bad;
            }
            out |= code << (8 * i + 2 * j);
          }
        }
        word[w] = out;
      }
    }
    uint4 o;
    o.x = word[0];
    o.y = word[1];
    o.z = word[2];
    o.w = word[3];
    reinterpret_cast<uint4*>(packed)[L] = o;
  }
  if (n_invalid != nullptr) {
    bad = wave_sum(bad);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(n_invalid, bad);
  }
}

// Quantizes one token row of length k (one workgroup of 256 threads).  Rows
// of up to kRegRow inputs stay in registers between the absmax and the
// rounding (one read of the row); longer rows are read twice.  Both passes
// take the same operations in the same precision: fp32 absmax, one correctly
// rounded 127 / a, an fp32 product, round half to even, clamp +-127.
constexpr int kRegVec = 8;                     // float4 per thread held
constexpr int64_t kRegRow = 256 * 4 * kRegVec;  // 8192 inputs

__device__ __forceinline__ void quant_row(const float* __restrict__ x,
                                          int64_t k, int8_t* __restrict__ xq,
                                          float* __restrict__ sa, int64_t row,
                                          float* part) {
  const float4* xr = reinterpret_cast<const float4*>(x + row * k);
  int32_t* qr = reinterpret_cast<int32_t*>(xq + row * k);
  const int64_t k4 = k >> 2;
  const int tid = threadIdx.x;
  float amax = 0.0f;
  float4 v[kRegVec];
  const bool in_regs = k <= kRegRow;  // uniform
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kRegVec; ++r) {
      const int64_t i = tid + 256 * r;
      v[r] = i < k4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[r].x), fabsf(v[r].y)),
                               fmaxf(fabsf(v[r].z), fabsf(v[r].w))));
    }
  } else {
    for (int64_t i = tid; i < k4; i += 256) {
      const float4 w = xr[i];
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)),
                               fmaxf(fabsf(w.z), fabsf(w.w))));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const QScale qs = quant_scale(amax);
  const float inv = qs.inv;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kRegVec; ++r) {
      const int64_t i = tid + 256 * r;
      if (i < k4) qr[i] = (int32_t)quant4(v[r], inv);
    }
  } else {
    for (int64_t i = tid; i < k4; i += 256) qr[i] = (int32_t)quant4(xr[i], inv);
  }
  if (tid == 0) sa[row] = qs.sa;
}

// One workgroup per token row.
__global__ __launch_bounds__(256) void quant_kernel(const float* __restrict__ x,
                                                    int64_t k,
                                                    int8_t* __restrict__ xq,
                                                    float* __restrict__ sa) {
  __shared__ float part[4];
  quant_row(x, k, xq, sa, blockIdx.x, part);
}

// Several quantizations in one launch: workgroup b takes the row
// b - first[j] of the job j with first[j] <= b < first[j + 1].
struct QuantJobs {
  const float* x[kMaxQuantJobs];
  int8_t* xq[kMaxQuantJobs];
  float* sa[kMaxQuantJobs];
  int64_t k[kMaxQuantJobs];
  int64_t first[kMaxQuantJobs + 1];
  int32_t count;
};

__global__ __launch_bounds__(256) void quant_many_kernel(QuantJobs jobs) {
  __shared__ float part[4];
  const int64_t b = blockIdx.x;
  int j = 0;
  while (j + 1 < jobs.count && jobs.first[j + 1] <= b) ++j;
  quant_row(jobs.x[j], jobs.k[j], jobs.xq[j], jobs.sa[j], b - jobs.first[j],
            part);
}

// RMSNorm then absmax quantization of one token row per wave (4 rows per
// workgroup).  The row's first 8 float4 per lane stay in registers across the
// three passes (sum of squares, normalized absmax, rounding); the rest of a
// longer row is read again for each pass.  The sum of squares follows the
// fixed order stated with sumsq4 in bt_internal.h.
constexpr int kNormHeld = 8;  // float4 per lane held in registers

__global__ __launch_bounds__(256) void norm_quant_kernel(
    const float* __restrict__ x, const float* __restrict__ g, int64_t m,
    int64_t k, float eps, int8_t* __restrict__ xq, float* __restrict__ sa,
    float* __restrict__ hout) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;  // wave-uniform; no workgroup barrier follows
  const float4* xr = reinterpret_cast<const float4*>(x + row * k);
  const float4* gr = reinterpret_cast<const float4*>(g);
  float4* hr = hout ? reinterpret_cast<float4*>(hout + row * k) : nullptr;
  int32_t* qr = reinterpret_cast<int32_t*>(xq + row * k);
  const int64_t n4 = k >> 2;
  constexpr int64_t kStep = 64 * kNormHeld;
  float4 v[kNormHeld];
  double ss = 0.0;
#pragma unroll
  for (int u = 0; u < kNormHeld; ++u) {
    const int64_t i = u * 64 + lane;
    v[u] = i < n4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (i < n4) ss = sumsq4(ss, v[u]);
  }
  for (int64_t b0 = kStep; b0 < n4; b0 += kStep)
#pragma unroll
    for (int u = 0; u < kNormHeld; ++u) {
      const int64_t i = b0 + u * 64 + lane;
      if (i < n4) ss = sumsq4(ss, xr[i]);
    }
  const float r = rms_scale(wave_sum_f64(ss), k, eps);
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < kNormHeld; ++u) {
    const int64_t i = u * 64 + lane;
    if (i < n4) {
      v[u] = rms_apply(v[u], r, gr[i]);
      amax = fmaxf(amax, absmax4(v[u]));
      if (hr) hr[i] = v[u];
    }
  }
  for (int64_t b0 = kStep; b0 < n4; b0 += kStep)
#pragma unroll
    for (int u = 0; u < kNormHeld; ++u) {
      const int64_t i = b0 + u * 64 + lane;
      if (i < n4) {
        const float4 hv = rms_apply(xr[i], r, gr[i]);
        amax = fmaxf(amax, absmax4(hv));
        if (hr) hr[i] = hv;
      }
    }
  const QScale qs = quant_scale(wave_max(amax));
#pragma unroll
  for (int u = 0; u < kNormHeld; ++u) {
    const int64_t i = u * 64 + lane;
    if (i < n4) qr[i] = (int32_t)quant4(v[u], qs.inv);
  }
  for (int64_t b0 = kStep; b0 < n4; b0 += kStep)
#pragma unroll
    for (int u = 0; u < kNormHeld; ++u) {
      const int64_t i = b0 + u * 64 + lane;
      if (i < n4) qr[i] = (int32_t)quant4(rms_apply(xr[i], r, gr[i]), qs.inv);
    }
  if (lane == 0) sa[row] = qs.sa;
}

}  // namespace

hipError_t launch_norm_quant(const float* x, const float* g, int64_t m,
                             int64_t k, float eps, int8_t* xq, float* sa,
                             float* h, hipStream_t s) {
  norm_quant_kernel<<<dim3((unsigned)((m + 3) / 4)), dim3(256), 0, s>>>(
      x, g, m, k, eps, xq, sa, h);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                       int32_t* n_invalid, hipStream_t s) {
  const int64_t total = (n + 63) / 64 * (k >> 6) * 64;
  const int64_t blocks = (total + 255) / 256;
  pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(t, n, k, total,
                                                           packed, n_invalid);
  return hipGetLastError();
}

hipError_t launch_quant(const float* x, int64_t m, int64_t k, int8_t* xq,
                        float* sa, hipStream_t s) {
  quant_kernel<<<dim3((unsigned)m), dim3(256), 0, s>>>(x, k, xq, sa);
  return hipGetLastError();
}

hipError_t launch_quant_many(const bt_quant_job* jobs, int32_t count,
                             hipStream_t s) {
  QuantJobs q;
  memset(&q, 0, sizeof(q));
  int64_t rows = 0;
  for (int32_t j = 0; j < count; ++j) {
    q.x[j] = jobs[j].x;
    q.xq[j] = jobs[j].x_q;
    q.sa[j] = jobs[j].s_a;
    q.k[j] = jobs[j].k;
    q.first[j] = rows;
    rows += jobs[j].m;
  }
  q.first[count] = rows;
  q.count = count;
  quant_many_kernel<<<dim3((unsigned)rows), dim3(256), 0, s>>>(q);
  return hipGetLastError();
}

}  // namespace bt
