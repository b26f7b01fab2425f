// Lookup-table ternary GEMV (one token): the table method of the pages' CPU
// kernels, kept to compare with the dot-product kernels on gfx950.
//
// "BitNet 1 位 LLM 独立推理引擎：位串行 GEMM 内核与 LUT 优化工程实践" (body,
// on kernel choice): TL1 turns every two weights into a 4-bit index and
// precomputed tables of the ternary combinations replace the per-weight
// decoding; TL2 does the same with three weights per 5-bit index.  Here the
// two weights of a pair are inputs k and k + 4, whose 2-bit codes sit side by
// side in one byte of the packed format (bits [4 h, 4 h + 4) of byte b of
// word g hold the codes of inputs 16 g + 8 h + b and 16 g + 8 h + b + 4), so
// the index is read straight from the packed weights: index = c0 + 4 c1 with
// codes c = trit + 1, 9 of its 16 values reachable.
//
// Mapping (wave64): a workgroup of 4, 8 or 16 waves owns one 64-row block,
// lane l of every wave owns row 64 b + l, and the waves split the block's
// chunks into contiguous ranges (as the dot-product kernel does, with the
// same number of waves).  A wave walks its range in tiles of 2 chunks (128
// inputs, 64 pairs): lane p first writes the 16 table entries
// (c0 - 1) x[k0] + (c1 - 1) x[k1] of pair p into the wave's LDS table, then
// every lane adds, for each of the 64 pairs, the entry its row's index
// selects.  Entry e of pair p sits at e * 66 + p (16-bit): 66
// entries span 33 banks, so the 16 indices of one pair fall in 16 different
// banks and the lanes' reads of one pair never conflict.  The sums are exact
// int32; the waves' partials meet in LDS and wave 0 applies the rescale.
#include "bt_internal.h"

namespace bt {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) int16_t* lds_i16_ptr;

constexpr int kStride = 66;     // 16-bit entries between two indices

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lut_kernel(Desc d) {
  __shared__ int16_t table[WAVES][16 * kStride];
  __shared__ int red[WAVES][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x;
  const int k = d.k;
  const int kc = k >> 6;
  const int c0 = kc * wave / WAVES;
  const int c1 = kc * (wave + 1) / WAVES;
  const v4u* wp =
      reinterpret_cast<const v4u*>(d.w + (size_t)rb * 16 * (size_t)k) + lane;
  const lds_i16_ptr t = (lds_i16_ptr)table[wave];
  // the pair this lane fills: chunk cc of the tile, word g, half h, byte b
  const int cc = lane >> 5, g = (lane >> 3) & 3, h = (lane >> 2) & 1,
            b = lane & 3;
  const int koff = 64 * cc + 16 * g + 8 * h + b;
  int acc = 0;
  for (int c = c0; c < c1; c += 2) {
    const int nch = min(2, c1 - c);
    // the tile's table; the wave's previous reads of it are done first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bool have = cc < nch;
    const int x0 = have ? (int)d.xq[64 * c + koff] : 0;
    const int x1 = have ? (int)d.xq[64 * c + koff + 4] : 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ca = e & 3, cb = e >> 2;
      const int v = (ca == 3 || cb == 3) ? 0 : (ca - 1) * x0 + (cb - 1) * x1;
      t[e * kStride + lane] = (int16_t)v;
    }
    // written and read by this wave only: LDS keeps its operations in order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int j = 0; j < nch; ++j) {
      const v4u wv = __builtin_nontemporal_load(wp + (size_t)(c + j) * 64);
      const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int idx = (words[gg] >> (8 * bb + 4 * hh)) & 15;
            const int pair = 32 * j + 8 * gg + 4 * hh + bb;
            acc += t[idx * kStride + pair];
          }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const int row = rb * 64 + lane;
    if (row < d.n) {
      int total = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) total += red[w][lane];
      if (d.acc != nullptr) d.acc[row] = total;
      d.y[row] = __fmul_rn(__fmul_rn((float)total, d.sw), d.sa[0]);
    }
  }
}

}  // namespace

hipError_t launch_lut(const Desc& d, hipStream_t s) {
  if (d.m != 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)d.nblk);
  // the dot-product kernel's choice of waves per row block
  switch (row_block_waves(d.nblk, d.kc)) {
    case 16: lut_kernel<16><<<grid, dim3(1024), 0, s>>>(d); break;
    case 8: lut_kernel<8><<<grid, dim3(512), 0, s>>>(d); break;
    default: lut_kernel<4><<<grid, dim3(256), 0, s>>>(d); break;
  }
  return hipGetLastError();
}

}  // namespace bt
