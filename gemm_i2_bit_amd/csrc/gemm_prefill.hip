// Ternary GEMM for many tokens (prefill) on int8 matrix cores
// (v_mfma_i32_32x32x32_i8, gfx950), activations staged through LDS.
//
// Once the 2-bit codes are expanded to int8 the ternary product is a dense
// integer contraction (bitnet.cpp CPU tutorial §1.1: each product with a
// trit is the activation, its negation or nothing, then accumulated), so at
// large m it is bound by the matrix cores, not by memory.  Codes c = trit + 1
// in {0, 1, 2} feed the matrix cores as they are; the per-token activation sum
// removes the +1 (sum (c - 1) q = sum c q - sum q), exact in int32.
//
// Workgroup tile: 128 tokens x 128 weight rows (two 64-row blocks of the
// packed layout), reduction in stages of 4 packed chunks (256 inputs).
//  * Activations: the 128 x 256 int8 stage is loaded cooperatively (128
//    bytes per thread) into one of two LDS buffers while the other is
//    consumed; one barrier per stage.  LDS rows are padded by 16 bytes.
//  * Weights: each wave owns one 64-row block (two 32-row MFMA tiles).  Lane
//    (h, i) reads 8 bytes of row i's 16-byte chunk: 32-bit words 2h and
//    2h + 1, i.e. inputs 64 c + 32 h + [0, 32).  Word s is expanded in
//    registers (shift and mask per 4 inputs) into the 16 int8 codes of
//    inputs 64 c + 32 h + 16 s + [0, 16): the A operand of MFMA step s.
//  * The B operand of step s is the same 16 inputs of token i, read from LDS
//    with one 128-bit load; the k assignment is identical on both sides, so
//    each MFMA step covers 32 distinct inputs (two groups h of 16).
//  * Output D[row][token] of a 32x32 tile sits in lane token + 32 ((row / 4)
//    % 2), register 4 (row / 8) + row % 4: each lane holds one token and 16
//    rows, stored as four 16-byte pieces.
#include "bt_internal.h"

namespace bt {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;          // tokens per workgroup tile
constexpr int CPS = 4;           // packed chunks (64 inputs each) per stage
constexpr int LDS_STRIDE = 64 * CPS + 16;  // bytes per token row of a stage

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

__device__ __forceinline__ void store_rows(const Desc& d, const v16i& c,
                                           int row0, int tok, int h, int qsum,
                                           float sa) {
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

// One workgroup tile: weight rows [128 rt, 128 rt + 128) x tokens
// [128 tt, 128 tt + 128).  Stages of CPS chunks (256 inputs): the next
// stage's loads (activations into registers, then LDS; weight words into
// registers) are issued before the current stage's 32 MFMAs per wave, which
// is long enough to cover an L2 round trip.
__device__ __forceinline__ void prefill_tile(const Desc& d, int rt, int tt,
                                             int8_t* lds) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int li = lane & 31;
  const int wm = wave >> 1;  // token half of the tile
  const int wn = wave & 1;   // row block of the tile
  const int k = d.k;
  const int kc = k >> 6;
  const int nst = (kc + CPS - 1) / CPS;
  const int blk = rt * 2 + wn;
  const bool blk_ok = blk < d.nblk;  // wave-uniform

  // weight words: row tile r2 of the block, row r2 * 32 + li, bytes 8h..8h+7
  // of each chunk
  const uint8_t* wrow0 = d.w + (size_t)(blk_ok ? blk : 0) * 16 * (size_t)k +
                         li * 16 + 8 * h;
  const uint8_t* wrow1 = wrow0 + 32 * 16;

  // cooperative activation load of a stage: token tid / 2, chunk parts
  // 32 (tid % 2) .. +32 of each of the CPS chunks
  const int tok_ld = tt * BM + (tid >> 1);
  const bool tok_ld_ok = tok_ld < d.m;
  const int8_t* qld =
      d.xq + (size_t)(tok_ld_ok ? tok_ld : 0) * k + (tid & 1) * 32;
  int8_t* lds_wr = lds + (tid >> 1) * LDS_STRIDE + (tid & 1) * 32;
  constexpr int kStage = BM * LDS_STRIDE;

  v16i acc[2][2];
#pragma unroll
  for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[r2][i] = v16i{0};
  int qsum[2] = {0, 0};

  v4i ga[CPS][2];
  uint2 w0[CPS], w1[CPS];
  auto load_stage = [&](int st) {
#pragma unroll
    for (int j = 0; j < CPS; ++j) {
      const int c = st * CPS + j;
      const bool ok = c < kc;
      ga[j][0] = ga[j][1] = v4i{0};
      w0[j] = w1[j] = make_uint2(0, 0);
      if (ok && tok_ld_ok) {
        ga[j][0] = *reinterpret_cast<const v4i*>(qld + (size_t)c * 64);
        ga[j][1] = *reinterpret_cast<const v4i*>(qld + (size_t)c * 64 + 16);
      }
      if (ok && blk_ok) {
        w0[j] = *reinterpret_cast<const uint2*>(wrow0 + (size_t)c * 1024);
        w1[j] = *reinterpret_cast<const uint2*>(wrow1 + (size_t)c * 1024);
      }
    }
  };
  auto store_stage = [&](int buf) {
    int8_t* nw = lds_wr + buf * kStage;
#pragma unroll
    for (int j = 0; j < CPS; ++j) {
      *reinterpret_cast<v4i*>(nw + j * 64) = ga[j][0];
      *reinterpret_cast<v4i*>(nw + j * 64 + 16) = ga[j][1];
    }
  };

  load_stage(0);
  store_stage(0);
  uint2 cw0[CPS], cw1[CPS];
#pragma unroll
  for (int j = 0; j < CPS; ++j) {
    cw0[j] = w0[j];
    cw1[j] = w1[j];
  }
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) load_stage(st + 1);
    // consume stage st
    const int8_t* lrd = lds + buf * kStage + (wm * 64 + li) * LDS_STRIDE;
#pragma unroll
    for (int j = 0; j < CPS; ++j) {
      if (st * CPS + j >= kc) break;  // uniform: ragged last stage
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4i b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          b[i] = *reinterpret_cast<const v4i*>(
              lrd + i * 32 * LDS_STRIDE + j * 64 + 16 * (2 * h + s));
          qsum[i] = sdot4(b[i].x, 0x01010101, qsum[i]);
          qsum[i] = sdot4(b[i].y, 0x01010101, qsum[i]);
          qsum[i] = sdot4(b[i].z, 0x01010101, qsum[i]);
          qsum[i] = sdot4(b[i].w, 0x01010101, qsum[i]);
        }
        if (blk_ok) {
          const v4i a0 = expand(s == 0 ? cw0[j].x : cw0[j].y);
          const v4i a1 = expand(s == 0 ? cw1[j].x : cw1[j].y);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            acc[0][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                a0, b[i], acc[0][i], 0, 0, 0);
            acc[1][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                a1, b[i], acc[1][i], 0, 0, 0);
          }
        }
      }
    }
    if (more) {
      store_stage(buf ^ 1);
#pragma unroll
      for (int j = 0; j < CPS; ++j) {
        cw0[j] = w0[j];
        cw1[j] = w1[j];
      }
    }
    __syncthreads();
  }

  if (!blk_ok) return;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // lanes li and li + 32 summed the two input halves of token li
    const int qs = qsum[i] + __shfl_xor(qsum[i], 32, 64);
    const int tok = tt * BM + wm * 64 + i * 32 + li;
    if (tok < d.m) {
      const float sa = d.sa[tok];
      store_rows(d, acc[0][i], blk * 64, tok, h, qs, sa);
      store_rows(d, acc[1][i], blk * 64 + 32, tok, h, qs, sa);
    }
  }
}

__global__ __launch_bounds__(256) void prefill_kernel(Desc d, int ntt) {
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * BM * LDS_STRIDE];
  const int u = blockIdx.x;
  prefill_tile(d, u / ntt, u % ntt, lds);
}

__global__ __launch_bounds__(256) void prefill_grouped_kernel(
    const Desc* __restrict__ descs, const Unit* __restrict__ units) {
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * BM * LDS_STRIDE];
  const Unit u = units[blockIdx.x];
  const Desc d = descs[u.prob];
  const int ntt = (d.m + BM - 1) / BM;
  prefill_tile(d, u.sub / ntt, u.sub % ntt, lds);
}

}  // namespace

int prefill_units(int64_t n, int64_t m) {
  return (int)(((n + 127) / 128) * ((m + BM - 1) / BM));
}

hipError_t launch_prefill(const Desc& d, hipStream_t s) {
  const int ntt = (d.m + BM - 1) / BM;
  const int units = prefill_units(d.n, d.m);
  prefill_kernel<<<dim3((unsigned)units), dim3(256), 0, s>>>(d, ntt);
  return hipGetLastError();
}

hipError_t launch_prefill_grouped(const Desc* descs, const Unit* units,
                                  int64_t count, hipStream_t s) {
  prefill_grouped_kernel<<<dim3((unsigned)count), dim3(256), 0, s>>>(descs,
                                                                     units);
  return hipGetLastError();
}

}  // namespace bt
