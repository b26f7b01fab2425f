// Ternary GEMM for many tokens (prefill) on int8 matrix cores
// (v_mfma_i32_32x32x32_i8, gfx950), operands staged through LDS by direct
// buffer-to-LDS loads.
//
// Once the 2-bit codes are expanded to int8 the ternary product is a dense
// integer contraction (bitnet.cpp CPU tutorial §1.1: each product with a
// trit is the activation, its negation or nothing, then accumulated), so at
// large m it is bound by the matrix cores, not by memory.  Codes c = trit + 1
// in {0, 1, 2} feed the matrix cores as they are; the per-token activation sum
// removes the +1 (sum (c - 1) q = sum c q - sum q), exact in int32.
//
// Workgroup tile: 256 weight rows (four 64-row blocks of the packed layout,
// one per wave) x 128 tokens.  The reduction runs in stages of 2 packed
// chunks (128 inputs) through a ring of 3 LDS slots: the loads of stage
// st + 2 are issued when stage st starts, so two stages of matrix-core work
// cover each load's latency.  One barrier per stage.
//  * Loads are buffer loads that write LDS directly (16 bytes per lane), with
//    no registers in between.  Their ranges end at the tile's last token and
//    at the block's last chunk, so tokens past m and weight words past the
//    row read as zero.  All variable offsets go in the range-checked offset.
//  * Activation slot: 128 token rows of 144 bytes (128 + 16 of padding).  Nine
//    is odd, so the matrix-core reads (one token per lane, 16 bytes at the
//    same column) meet no bank conflicts, and every read offset within a
//    stage is an immediate.
//  * Weight slot: per wave, the block's two 1 KiB chunks copied as they are.
//  * Matrix-core operands: lane (h, i) takes 8 bytes of row i's 16-byte chunk,
//    32-bit words 2h and 2h + 1 (inputs 64 c + 32 h + [0, 32)).  Word s is
//    expanded in registers (shift and mask per 4 inputs) into the 16 int8
//    codes of inputs 64 c + 32 h + 16 s + [0, 16): the A operand of step s;
//    it feeds four MFMAs (the wave's four 32-token tiles).  The B operand is
//    the same 16 inputs of token i, one 128-bit LDS read; the k assignment is
//    identical on both sides, so each step covers 32 distinct inputs.
//  * Activation sums: each wave visits the four token tiles starting at its
//    own, adds up the B operands of its own tile as they pass (4 dot4 per
//    step) and shares them through LDS at the end.
//  * Ragged k (an odd number of chunks): the second chunk of the last stage
//    has zero weight words (out of range) and is left out of the activation
//    sums.  A block past the last row block reads zeros and is never stored.
//  * Output D[row][token] of a 32x32 tile sits in lane token + 32 ((row / 4)
//    % 2), register 4 (row / 8) + row % 4: each lane holds one token and 16
//    rows, stored as four 16-byte pieces.
#include <type_traits>

#include "bt_internal.h"

namespace bt {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) float* gfloat_ptr;
typedef __attribute__((address_space(1))) int32_t* gint_ptr;
typedef const __attribute__((address_space(1))) float* gcfloat_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BM = 128;   // tokens per workgroup tile
constexpr int BLK = 4;    // 64-row blocks per tile, one per wave
constexpr int CPS = 2;    // packed chunks per stage
constexpr int NS = 3;     // LDS ring slots
constexpr int kRowGran = CPS * 4 + 1;  // 16-byte granules per token row,
                                       // one of them padding
constexpr int kRow = kRowGran * 16;    // 144 bytes
constexpr int kActSlot = BM * kRow;    // 18 KiB
constexpr int kWSlot = BLK * CPS * 1024;  // 8 KiB
// direct loads filling one activation slot: 64 granules each, spread over
// the waves (the last round repeats loads of waves 0 and 1)
constexpr int kActLoads = (BM * kRowGran + 63) / 64;        // 18
constexpr int kActDma = (kActLoads + BLK - 1) / BLK;        // 5 per wave
constexpr int kDmaPerStage = kActDma + CPS;  // loads per wave per stage
// Buffer resource word 3 for raw (untyped, unswizzled) gfx9 buffer loads.
constexpr int kRsrcFlags = 0x00020000;

static_assert(kActLoads == 18 && kActDma == 5 && kDmaPerStage == 7,
              "stage shape");

// s_waitcnt immediate: vmcnt(v) and lgkmcnt(0); expcnt not waited on
constexpr int waitcnt_vm(int v) {
  return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (0 << 8);
}

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
  const gfloat_ptr y = (gfloat_ptr)d.y + base;
  const gint_ptr acc = d.acc ? (gint_ptr)d.acc + base : nullptr;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int row = row0 + 8 * g + 4 * h;  // 4 consecutive rows
    int a[4];
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = c[4 * g + r] - qsum;
      v[r] = __fmul_rn(__fmul_rn((float)a[r], d.sw), sa);
    }
    if ((d.n & 3) == 0 && row + 3 < d.n) {
      *reinterpret_cast<__attribute__((address_space(1))) v4f*>(y + row) =
          v4f{v[0], v[1], v[2], v[3]};
      if (acc)
        *reinterpret_cast<__attribute__((address_space(1))) v4i*>(acc + row) =
            v4i{a[0], a[1], a[2], a[3]};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (row + r < d.n) {
          y[row + r] = v[r];
          if (acc) acc[row + r] = a[r];
        }
      }
    }
  }
}

// The LDS ring: one array per slot and operand.  Separate arrays let the
// compiler tell the slots apart, so a read of one slot does not wait for the
// direct loads still in flight into the others.
struct Ring {
  int8_t* act[NS];  // kActSlot bytes each
  int8_t* wts[NS];  // kWSlot bytes each
};

// One stage of matrix-core work from one ring slot.  `ones1` is 0x01010101,
// or 0 when the stage's second chunk lies past the row (odd kc): its weight
// words read as zero, so only the activation sums have to skip it.
// B operand i comes from token tile (i + wave) mod 4 (byte offset bread[i]),
// so that B operand 0 is the wave's own tile for the activation sums.
__device__ __forceinline__ void compute_stage(const int8_t* act,
                                              const int8_t* wslot,
                                              const int (&bread)[4],
                                              int wread, int ones1,
                                              v16i (&acc)[2][4],
                                              int& tsum_part) {
#pragma unroll
  for (int j = 0; j < CPS; ++j) {
    const int ones = j == 0 ? 0x01010101 : ones1;
    const v2i w0 = *reinterpret_cast<const v2i*>(wslot + j * 1024 + wread);
    const v2i w1 =
        *reinterpret_cast<const v2i*>(wslot + j * 1024 + wread + 512);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b[i] = *reinterpret_cast<const v4i*>(act + bread[i] + 64 * j + 16 * s);
      const v4i a0 = expand((uint32_t)(s == 0 ? w0.x : w0.y));
      const v4i a1 = expand((uint32_t)(s == 0 ? w1.x : w1.y));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[0][i] =
            __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b[i], acc[0][i], 0, 0, 0);
        acc[1][i] =
            __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b[i], acc[1][i], 0, 0, 0);
      }
      tsum_part = sdot4(b[0].x, ones, tsum_part);
      tsum_part = sdot4(b[0].y, ones, tsum_part);
      tsum_part = sdot4(b[0].z, ones, tsum_part);
      tsum_part = sdot4(b[0].w, ones, tsum_part);
    }
  }
}

// One workgroup tile: weight rows [256 rt, 256 rt + 256) x tokens
// [128 tt, 128 tt + 128).
__device__ __forceinline__ void prefill_tile(const Desc& d, int rt, int tt,
                                             const Ring& ring, int* tsum) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int li = lane & 31;
  const int k = d.k;
  const int kc = k >> 6;
  const int nst = (kc + CPS - 1) / CPS;
  const int blk = rt * BLK + wave;
  const bool blk_ok = blk < d.nblk;  // wave-uniform

  // weight loads: the wave's block, 1 KiB per chunk, lane = 16-byte row piece
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(d.w + (size_t)(blk_ok ? blk : 0) * 16 * (size_t)k), 0,
      blk_ok ? 16 * k : 0, kRsrcFlags);
  // activation loads: load q fills slot granules 64 q + lane, granule g of
  // the slot being byte 16 (g % 9) of token g / 9 (the ninth is padding and
  // gets a copy of the eighth).  Wave w issues loads q = w + 4 r.
  const int tok0 = tt * BM;
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(d.xq + (size_t)tok0 * k), 0, min(BM, d.m - tok0) * k,
      kRsrcFlags);
  int av[kActDma];
  int aq[kActDma];  // load index q (uniform)
#pragma unroll
  for (int r = 0; r < kActDma; ++r) {
    int q = wave + BLK * r;
    if (q >= kActLoads) q -= 2;  // repeat a load of waves 0 / 1
    aq[r] = q;
    const int g = q * 64 + lane;
    const int t = g / kRowGran;
    const int x = min(g % kRowGran, kRowGran - 2);
    av[r] = t * k + x * 16;
  }

  // loads of stage st into one ring slot
  auto issue = [&](int8_t* act, int8_t* wts, int st) {
    const int c0 = st * CPS;
#pragma unroll
    for (int r = 0; r < kActDma; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ar, (lds_ptr)(act + aq[r] * 1024), 16, av[r] + c0 * 64, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CPS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_ptr)(wts + (wave * CPS + j) * 1024), 16,
          lane * 16 + (c0 + j) * 1024, 0, 0, 0);
  };

  // matrix-core reads: B operand i is token (32 ((i + wave) % 4) + li),
  // inputs 64 j + 32 h + 16 s + [0, 16) of the stage
  int bread[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bread[i] = (32 * ((i + wave) & 3) + li) * kRow + 32 * h;
  const int wread = wave * CPS * 1024 + li * 16 + 8 * h;

  v16i acc[2][4];
#pragma unroll
  for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r2][i] = v16i{0};
  int tsum_part = 0;

  // Prologue: stages 0 .. NS-2 in flight.  Every stage issues one more (past
  // the end they read out of range or unused rows and are never consumed),
  // so exactly NS-2 stages are younger than the one awaited.
  static_assert(NS == 3, "the stage loop below is unrolled for 3 slots");
  issue(ring.act[0], ring.wts[0], 0);
  issue(ring.act[1], ring.wts[1], 1);
  // stage st from slot S; its successor's successor goes into slot S + 2
  const int nfull = kc / CPS;  // full stages; an odd kc adds one more
  auto stage = [&](auto slot_tag, int st) {
    constexpr int S = decltype(slot_tag)::value;
    constexpr int N = (S + NS - 1) % NS;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * kDmaPerStage));
    __builtin_amdgcn_s_barrier();
    issue(ring.act[N], ring.wts[N], st + NS - 1);
    compute_stage(ring.act[S], ring.wts[S], bread, wread,
                  st < nfull ? 0x01010101 : 0, acc, tsum_part);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  int st = 0;
  for (; st + NS <= nst; st += NS) {
    stage(S0{}, st);
    stage(S1{}, st + 1);
    stage(S2{}, st + 2);
  }
  if (st < nst) stage(S0{}, st);
  if (st + 1 < nst) stage(S1{}, st + 1);
  // drain the loads issued past the end before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // activation sums of token tile `wave`: lanes li and li + 32 hold the two
  // input halves of token 32 wave + li
  const int ts = tsum_part + __shfl_xor(tsum_part, 32, 64);
  if (h == 0) tsum[wave * 32 + li] = ts;
  __syncthreads();

  if (!blk_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tl = 32 * ((i + wave) & 3) + li;  // token within the tile
    const int tok = tok0 + tl;
    if (tok < d.m) {
      const int qs = tsum[tl];
      const float sa = *((gcfloat_ptr)d.sa + tok);
      store_rows(d, acc[0][i], blk * 64, tok, h, qs, sa);
      store_rows(d, acc[1][i], blk * 64 + 32, tok, h, qs, sa);
    }
  }
}

#define BT_PREFILL_LDS                                                \
  __shared__ __attribute__((aligned(1024))) int8_t a0[kActSlot];     \
  __shared__ __attribute__((aligned(1024))) int8_t a1[kActSlot];     \
  __shared__ __attribute__((aligned(1024))) int8_t a2[kActSlot];     \
  __shared__ __attribute__((aligned(1024))) int8_t w0[kWSlot];       \
  __shared__ __attribute__((aligned(1024))) int8_t w1[kWSlot];       \
  __shared__ __attribute__((aligned(1024))) int8_t w2[kWSlot];       \
  __shared__ int tsum[BM];                                           \
  const Ring ring = {{a0, a1, a2}, {w0, w1, w2}}

__global__ __launch_bounds__(256, 2) void prefill_kernel(Desc d, int ntt) {
  BT_PREFILL_LDS;
  const int u = blockIdx.x;
  prefill_tile(d, u / ntt, u % ntt, ring, tsum);
}

__global__ __launch_bounds__(256, 2) void prefill_grouped_kernel(
    const Desc* __restrict__ descs, const Unit* __restrict__ units) {
  BT_PREFILL_LDS;
  const Unit u = units[blockIdx.x];
  const Desc d = descs[u.prob];
  const int ntt = (d.m + BM - 1) / BM;
  prefill_tile(d, u.sub / ntt, u.sub % ntt, ring, tsum);
}
#undef BT_PREFILL_LDS

}  // namespace

hipError_t launch_prefill(const Desc& d, hipStream_t s) {
  const int ntt = (d.m + BM - 1) / BM;
  const int64_t units = kind_units(kKindPrefill, d.n, d.m);
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
