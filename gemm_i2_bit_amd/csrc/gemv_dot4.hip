// Ternary GEMV / very skinny GEMM (m <= 4 tokens) with packed int8 dot
// products (v_dot4_i32_i8).
//
// The product is memory bound: a weight is 2 bits and is used m <= 4 times,
// so the kernel streams the packed weights once at HBM speed ("1bit-systems"
// page, section "性能实测：92%的内存带宽利用率": the ternary GEMV saturates
// memory and only fewer bytes make it faster).  Multiplying by -1/0/+1 is a
// sign test plus accumulation (bitnet.cpp CPU tutorial §1.1); here it is done
// exactly in int32 with the code-offset identity
//     sum_k (c_k - 1) q_k = sum_k c_k q_k - sum_k q_k,   c_k = trit + 1,
// so raw 2-bit codes feed v_dot4 directly and one activation sum per token is
// subtracted at the end.
//
// Single-problem mapping (gfx950, wave64): a workgroup of WAVES waves owns
// one 64-row block; lane l of every wave owns row 64 b + l, and the waves
// split the block's 16-byte chunks (64 inputs each) into WAVES contiguous
// ranges.  A matrix with few row blocks gets more waves per block (4, 8 or
// 16, at least 4 chunks each), so that it still puts enough loads in flight:
// 2560 x 6912 has only 40 row blocks.  For a chunk, the
// 64 lanes read one contiguous KiB (one 128-bit load each) and all need the
// same 64 activation bytes per token, which are wave-uniform and live in
// scalar registers.  Within a 32-bit word of codes, the four 2-bit fields are
// masked in place: field j holds 4^j * code, so each field has its own int32
// accumulator and the fields are combined with exact shifts at the end.
// Partial sums of the waves meet in LDS; wave 0 applies the rescale.
// Grouped calls use the persistent streaming kernel instead.
#include "bt_internal.h"

namespace bt {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int TOK, int WAVES>
__device__ __forceinline__ void dot4_block(const Desc& d, int rb,
                                           int (*red)[TOK][64]) {
  const int lane = threadIdx.x & 63;
  // wave index in a scalar register: the compiler then treats the chunk range
  // and every activation address as wave-uniform (scalar loads).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = d.k;
  const int kc = k >> 6;
  const int c0 = kc * wave / WAVES;
  const int c1 = kc * (wave + 1) / WAVES;
  const int kq = k >> 2;  // activation row length in 32-bit words

  const v4u* wp =
      reinterpret_cast<const v4u*>(d.w + (size_t)rb * 16 * (size_t)k) + lane;
  const int* q = reinterpret_cast<const int*>(d.xq);

  int a0[TOK], a1[TOK], a2[TOK], a3[TOK];
#pragma unroll
  for (int t = 0; t < TOK; ++t) a0[t] = a1[t] = a2[t] = a3[t] = 0;

#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    // streamed once: non-temporal loads keep the weights from displacing
    // reusable lines in the caches
    const v4u wv = __builtin_nontemporal_load(wp + (size_t)c * 64);
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = (int)(words[w] & 0x03030303u);
      const int e1 = (int)(words[w] & 0x0C0C0C0Cu);
      const int e2 = (int)(words[w] & 0x30303030u);
      const int e3 = (int)((words[w] >> 6) & 0x03030303u);
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        const int* qc = q + t * kq + c * 16 + 4 * w;
        a0[t] = sdot4(e0, qc[0], a0[t]);
        a1[t] = sdot4(e1, qc[1], a1[t]);
        a2[t] = sdot4(e2, qc[2], a2[t]);
        a3[t] = sdot4(e3, qc[3], a3[t]);
      }
    }
  }

  // Sum of the activations over this wave's inputs, per token (wave-wide).
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    int s = 0;
    const int* qt = q + t * kq + c0 * 16;
    const int nw = (c1 - c0) * 16;
    for (int i = lane; i < nw; i += 64) s = sdot4(qt[i], 0x01010101, s);
    s = wave_sum(s);
    red[wave][t][lane] = a0[t] + (a1[t] >> 2) + (a2[t] >> 4) + a3[t] - s;
  }
  __syncthreads();
  if (wave == 0) {
    const int row = rb * 64 + lane;
    if (row < d.n) {
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        int acc = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) acc += red[w][t][lane];
        const size_t o = (size_t)t * d.n + row;
        if (d.acc != nullptr) d.acc[o] = acc;
        d.y[o] = __fmul_rn(__fmul_rn((float)acc, d.sw), d.sa[t]);
      }
    }
  }
}

template <int TOK, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void dot4_kernel(Desc d) {
  __shared__ int red[WAVES][TOK][64];
  dot4_block<TOK, WAVES>(d, blockIdx.x, red);
}

template <int WAVES>
hipError_t launch_waves(const Desc& d, hipStream_t s) {
  const dim3 grid((unsigned)d.nblk), block(64 * WAVES);
  switch (d.m) {
    case 1: dot4_kernel<1, WAVES><<<grid, block, 0, s>>>(d); break;
    case 2: dot4_kernel<2, WAVES><<<grid, block, 0, s>>>(d); break;
    case 3: dot4_kernel<3, WAVES><<<grid, block, 0, s>>>(d); break;
    case 4: dot4_kernel<4, WAVES><<<grid, block, 0, s>>>(d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dot4(const Desc& d, hipStream_t s) {
  switch (row_block_waves(d.nblk, d.kc)) {
    case 16: return launch_waves<16>(d, s);
    case 8: return launch_waves<8>(d, s);
    default: return launch_waves<4>(d, s);
  }
}

}  // namespace bt
