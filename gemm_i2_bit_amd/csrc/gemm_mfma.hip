// Ternary GEMM for m > 4 tokens on int8 matrix cores
// (v_mfma_i32_32x32x32_i8, gfx950).
//
// The ternary product is a dense integer contraction once the 2-bit codes are
// expanded to int8 (bitnet.cpp CPU tutorial §1.1: the product of a trit and an
// activation is the activation, its negation or nothing, accumulated).  The
// kernel expands codes c = trit + 1 in {0, 1, 2} in registers (one shift and
// one mask per 4 inputs) and feeds them to the matrix cores as they are; the
// code-offset identity  sum (c - 1) q = sum c q - sum q  removes the +1 with
// one per-token activation sum, exact in int32.
//
// Mapping: each wave owns a 64-row x 32-token output tile (two 32x32 MFMA
// tiles stacked in rows) over the full reduction length; a workgroup holds 4
// such waves, consecutive in the work order (row blocks, then token tiles),
// so neighbouring waves share activations and weights through the L1 cache.
// MFMA operand layout (32x32x32, 16 int8 per lane): lane l supplies row
// (l % 32) of A and column (l % 32) of B, for one of two 16-input groups
// (l / 32).  Lane (h, i) loads 16-byte chunk 2p + h of weight row i, i.e.
// inputs [64 (2p + h), +64); its 32-bit word s gives the 16 codes of inputs
// 64 (2p + h) + 16 s + [0, 16), which pair with 16 contiguous activation
// bytes of token i for MFMA number s.  Output D[row][token] sits in lane
// token + 32 ((row / 4) % 2), register 4 (row / 8) + row % 4.
#include "bt_internal.h"

namespace bt {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ v4i expand(uint32_t word) {
  v4i a;
  a.x = (int)(word & 0x03030303u);
  a.y = (int)((word >> 2) & 0x03030303u);
  a.z = (int)((word >> 4) & 0x03030303u);
  a.w = (int)((word >> 6) & 0x03030303u);
  return a;
}

__device__ __forceinline__ void store_tile(const Desc& d, const v16i& c,
                                           int row0, int tok, int h, int qsum,
                                           bool tok_ok) {
  if (!tok_ok) return;
  const float sa = d.sa[tok];
  const size_t base = (size_t)tok * d.n;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int row = row0 + 8 * g + 4 * h;  // 4 consecutive rows
    int a[4];
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = c[4 * g + r] - qsum;
      y[r] = __fmul_rn(__fmul_rn((float)a[r], d.sw), sa);
    }
    if ((d.n & 3) == 0 && row + 3 < d.n) {
      *reinterpret_cast<float4*>(d.y + base + row) =
          make_float4(y[0], y[1], y[2], y[3]);
      if (d.acc != nullptr)
        *reinterpret_cast<int4*>(d.acc + base + row) =
            make_int4(a[0], a[1], a[2], a[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (row + r < d.n) {
          d.y[base + row + r] = y[r];
          if (d.acc != nullptr) d.acc[base + row + r] = a[r];
        }
      }
    }
  }
}

// One wave: rows [64 rb, 64 rb + 64) x tokens [32 tt, 32 tt + 32).
__device__ __forceinline__ void mfma_wave(const Desc& d, int rb, int tt) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int li = lane & 31;
  const int k = d.k;
  const int kc = k >> 6;
  const int tok = tt * 32 + li;
  const bool tok_ok = tok < d.m;

  const uint8_t* wblk = d.w + (size_t)rb * 16 * (size_t)k;
  const int8_t* qrow = d.xq + (size_t)(tok_ok ? tok : 0) * k;

  v16i c0 = {0}, c1 = {0};
  int qsum = 0;
  const int np = (kc + 1) >> 1;
#pragma unroll 2
  for (int p = 0; p < np; ++p) {
    const int ch = 2 * p + h;
    const bool ok = ch < kc;
    uint4 wa = make_uint4(0, 0, 0, 0), wb = make_uint4(0, 0, 0, 0);
    v4i q[4] = {{0}, {0}, {0}, {0}};
    if (ok) {
      wa = *reinterpret_cast<const uint4*>(wblk + (size_t)ch * 1024 + li * 16);
      wb = *reinterpret_cast<const uint4*>(wblk + (size_t)ch * 1024 +
                                           (32 + li) * 16);
      if (tok_ok) {
        const v4i* qp = reinterpret_cast<const v4i*>(qrow + (size_t)ch * 64);
#pragma unroll
        for (int s = 0; s < 4; ++s) q[s] = qp[s];
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qsum = sdot4(q[s].x, 0x01010101, qsum);
      qsum = sdot4(q[s].y, 0x01010101, qsum);
      qsum = sdot4(q[s].z, 0x01010101, qsum);
      qsum = sdot4(q[s].w, 0x01010101, qsum);
    }
    const uint32_t wA[4] = {wa.x, wa.y, wa.z, wa.w};
    const uint32_t wB[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(expand(wA[s]), q[s], c0, 0, 0,
                                                 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(expand(wB[s]), q[s], c1, 0, 0,
                                                 0);
    }
  }
  // Lanes li and li + 32 summed the two halves of token li's activations.
  qsum += __shfl_xor(qsum, 32, 64);
  store_tile(d, c0, rb * 64, tok, h, qsum, tok_ok);
  store_tile(d, c1, rb * 64 + 32, tok, h, qsum, tok_ok);
}

__global__ __launch_bounds__(256) void mfma_kernel(Desc d, int64_t units) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t u = (int64_t)blockIdx.x * 4 + wave;
  if (u >= units) return;
  mfma_wave(d, (int)(u / d.ntt), (int)(u % d.ntt));
}

__global__ __launch_bounds__(256) void mfma_grouped_kernel(
    const Desc* __restrict__ descs, const Unit* __restrict__ units,
    int64_t count) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  if (idx >= count) return;
  const Unit u = units[idx];
  const Desc d = descs[u.prob];
  mfma_wave(d, u.sub / d.ntt, u.sub % d.ntt);
}

}  // namespace

hipError_t launch_mfma(const Desc& d, hipStream_t s) {
  const int64_t units = (int64_t)d.nblk * d.ntt;
  mfma_kernel<<<dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s>>>(d,
                                                                      units);
  return hipGetLastError();
}

hipError_t launch_mfma_grouped(const Desc* descs, const Unit* units,
                               int64_t count, hipStream_t s) {
  mfma_grouped_kernel<<<dim3((unsigned)((count + 3) / 4)), dim3(256), 0, s>>>(
      descs, units, count);
  return hipGetLastError();
}

}  // namespace bt
