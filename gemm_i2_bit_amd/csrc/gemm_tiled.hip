// Ternary GEMM for m > 4 tokens on int8 matrix cores
// (v_mfma_i32_32x32x32_i8, gfx950), operands staged through LDS by direct
// buffer-to-LDS loads.
//
// Once the 2-bit codes are expanded to int8 the ternary product is a dense
// integer contraction (bitnet.cpp CPU tutorial §1.1: each product with a
// trit is the activation, its negation or nothing, then accumulated).  Codes
// c = trit + 1 in {0, 1, 2} feed the matrix cores as they are; the per-token
// activation sum removes the +1 (sum (c - 1) q = sum c q - sum q), exact in
// int32.  Skinny token counts (up to 64) stay bound by the weight stream from
// HBM; prefill-sized ones (128-token tiles) by the matrix cores.
//
// Workgroup tile: 256 weight rows (four 64-row blocks of the packed layout,
// one per wave) x BM tokens (32, 64 or 128).  The reduction runs in stages of
// 2 packed chunks (128 inputs) through a ring of NS LDS slots: the loads of
// stage st + NS - 1 are issued when stage st starts, so NS - 1 stages of work
// cover each load's latency.  One barrier per stage.
//  * Loads are buffer loads that write LDS directly (16 bytes per lane), with
//    no registers in between.  Their ranges end at the tile's last token and
//    at the block's last chunk, so tokens past m and weight words past the
//    row read as zero.  All variable offsets go in the range-checked offset.
//  * Activation slot: BM token rows of 144 bytes (128 + 16 of padding).  Nine
//    is odd, so the matrix-core reads (one token per lane, 16 bytes at the
//    same column) meet no bank conflicts, and every read offset within a
//    stage is an immediate.
//  * Weight slot: per wave, the block's two 1 KiB chunks copied as they are.
//  * Each slot is an LDS array of its own, so the compiler can tell them apart
//    and a read of one slot does not wait for the loads into the others.
//  * Matrix-core operands: lane (h, i) takes 8 bytes of row i's 16-byte chunk,
//    32-bit words 2h and 2h + 1 (inputs 64 c + 32 h + [0, 32)).  Word s is
//    expanded in registers (shift and mask per 4 inputs) into the 16 int8
//    codes of inputs 64 c + 32 h + 16 s + [0, 16): the A operand of step s;
//    it feeds one MFMA per 32-token tile of the wave.  The B operand is the
//    same 16 inputs of token i, one 128-bit LDS read; the k assignment is
//    identical on both sides, so each step covers 32 distinct inputs.
//  * Activation sums: wave w visits its token tiles starting at tile w mod NB
//    and adds up the B operands of that first tile as they pass (4 dot4 per
//    step); the sums go through LDS to the epilogue.
//  * Ragged k (an odd number of chunks): the second chunk of the last stage
//    has zero weight words (out of range) and is left out of the activation
//    sums.  A block past the last row block reads zeros and is never stored.
//  * Output D[row][token] of a 32x32 tile sits in lane token + 32 ((row / 4)
//    % 2), register 4 (row / 8) + row % 4: each lane holds one token and 16
//    rows.  The epilogue transposes them through LDS so that every token's
//    64 rows of a block go out as one 256-byte segment.
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

constexpr int BLK = 4;                 // 64-row blocks per tile, one per wave
constexpr int CPS = 2;                 // packed chunks per stage
constexpr int kRowGran = CPS * 4 + 1;  // 16-byte granules per token row,
                                       // one of them padding
constexpr int kRow = kRowGran * 16;    // 144 bytes
constexpr int kWSlot = BLK * CPS * 1024;  // 8 KiB
// Buffer resource word 3 for raw (untyped, unswizzled) gfx9 buffer loads.
constexpr int kRsrcFlags = 0x00020000;

template <int BM_, int NS_, bool RegW_, int BPW_ = 1>
struct Cfg {
  static constexpr int BM = BM_;       // tokens per workgroup tile
  static constexpr int NB = BM / 32;   // 32-token MFMA tiles per wave
  static constexpr int NS = NS_;       // LDS ring slots
  // weight words go from memory straight to registers (else through LDS)
  static constexpr bool kRegW = RegW_;
  // 64-row blocks per wave: the workgroup tile covers kRows weight rows, and
  // each activation byte brought into LDS serves BPW blocks of every wave
  static constexpr int BPW = BPW_;
  static constexpr int kRows = 64 * BLK * BPW;
  static_assert(BPW == 1 || kRegW, "several blocks per wave: weights in "
                                   "registers");
  // activation slot, rounded up to whole 1 KiB loads
  static constexpr int kActSlot = (BM * kRow + 1023) / 1024 * 1024;
  // direct loads filling one activation slot, 64 granules each, spread over
  // the waves (extra rounds repeat the last load)
  static constexpr int kActLoads = (BM * kRowGran + 63) / 64;
  static constexpr int kActDma = (kActLoads + BLK - 1) / BLK;
  // memory instructions per wave per stage, in issue order: activation
  // loads, then weight loads (into LDS, or into registers)
  static constexpr int kWLoads = kRegW ? 2 * BPW : CPS;
  static constexpr int kPerStage = kActDma + kWLoads;
  // at the start of a stage, the loads younger than its activation loads:
  // its own weight loads when they go to registers (the compiler waits for
  // those where they are used), and NS - 2 whole stages
  static constexpr int kYounger = (NS - 2) * kPerStage + (kRegW ? kWLoads : 0);
  static_assert(kActLoads * 1024 <= kActSlot, "slot holds every load");
  static_assert(kYounger < 64, "vmcnt range");
};
using CfgS32 = Cfg<32, 4, true>;
using CfgS64 = Cfg<64, 4, true, 2>;
using CfgP128 = Cfg<128, 3, false>;
// the plans count work units with the same tile heights
static_assert(CfgS32::kRows == tile_rows(32) && CfgS64::kRows == tile_rows(64) &&
                  CfgP128::kRows == tile_rows(128),
              "tile rows of the plans");

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

// One 16-byte piece per lane from buffer [base, base + bytes) at byte offset
// voff (range-checked: past the end reads zero) straight into LDS at
// lds + 16 lane.  `lds` is wave-uniform.
__device__ __forceinline__ void load_lds16(const void* base, int bytes,
                                           int8_t* lds, int voff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(base), 0, bytes, kRsrcFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, 0, 0, 0);
}

// Ring slot S of a configuration: one LDS array per slot and operand.
template <class C, int S>
__device__ __forceinline__ int8_t* act_slot() {
  __shared__ __attribute__((aligned(1024))) int8_t buf[C::kActSlot];
  return buf;
}
template <class C, int S>
__device__ __forceinline__ int8_t* wts_slot() {
  __shared__ __attribute__((aligned(1024))) int8_t buf[kWSlot];
  return buf;
}

template <class C>
__device__ __forceinline__ int* tsum_array() {
  __shared__ int buf[C::BM];
  return buf;
}

// Output staging of the epilogue: a wave's accumulators hold one token per
// lane and 16 rows per register set, so direct stores would scatter 16-byte
// pieces over 32 token rows.  Instead each wave passes TP tokens at a time
// through an LDS region of its own (rows of one token contiguous, rows padded
// to 272 bytes so that both the writes and the reads are free of bank
// conflicts) and stores every token's 64 rows as one 256-byte segment (16
// lanes x 16 bytes).  The region reuses the ring, which is idle by then.
constexpr int kEpRow = 272;  // bytes per token in the staging region

// 16 bytes of outputs (rows row .. row + 3 of token `tok`) from one lane.
// Outputs are written once and not read back by the launch.  NT: a
// non-temporal store, for the staged epilogue whose 16 lanes write a token's
// 256 contiguous bytes at once (measured 2 us faster on the M=512 layer);
// direct stores, which cover 32 bytes of a token per instruction, go through
// the L2 so that the pieces of a segment merge there before they reach
// memory (non-temporal ones were 6-9 % slower at 3 and 16 tokens).
template <typename T, bool NT>
__device__ __forceinline__ void store_row16(T* out, int n, int tok, int row,
                                            const int8_t* src) {
  T* dst = out + (size_t)tok * n + row;
  typedef __attribute__((address_space(1))) v4i* gv4i_ptr;
  if ((n & 3) == 0 && row + 3 < n) {
    const v4i v = *reinterpret_cast<const v4i*>(src);
    const gv4i_ptr p =
        reinterpret_cast<gv4i_ptr>((__attribute__((address_space(1))) T*)dst);
    if constexpr (NT)
      __builtin_nontemporal_store(v, p);
    else
      *p = v;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < n)
        ((__attribute__((address_space(1))) T*)dst)[r] =
            reinterpret_cast<const T*>(src)[r];
  }
}

// One stage of matrix-core work from one ring slot.  `ones1` is 0x01010101,
// or 0 when the stage's second chunk lies past the row (odd kc): its weight
// words read as zero, so only the activation sums have to skip it.
template <class C>
__device__ __forceinline__ void compute_stage(const int8_t* act,
                                              const int8_t* wslot,
                                              const int (&bread)[C::NB],
                                              int wread, int ones1,
                                              v16i (&acc)[2][C::NB],
                                              int& tsum_part) {
#pragma unroll
  for (int j = 0; j < CPS; ++j) {
    const int ones = j == 0 ? 0x01010101 : ones1;
    const v2i w0 = *reinterpret_cast<const v2i*>(wslot + j * 1024 + wread);
    const v2i w1 =
        *reinterpret_cast<const v2i*>(wslot + j * 1024 + wread + 512);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i b[C::NB];
#pragma unroll
      for (int i = 0; i < C::NB; ++i)
        b[i] = *reinterpret_cast<const v4i*>(act + bread[i] + 64 * j + 16 * s);
      const v4i a0 = expand((uint32_t)(s == 0 ? w0.x : w0.y));
      const v4i a1 = expand((uint32_t)(s == 0 ? w1.x : w1.y));
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
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

// One stage with weight words in registers: for each of the wave's blocks
// lane (h, i) holds the 16-byte chunk 2 p + h of rows i and 32 + i (w[.][0],
// w[.][1]); word s gives the A operands of step s, inputs 64 h + 16 s +
// [0, 16) of the stage, and one B operand read from LDS serves every block.
// `ones` is 0 for lanes whose chunk lies past the row (odd kc), else
// 0x01010101.
template <class C>
__device__ __forceinline__ void compute_stage_reg(const int8_t* act,
                                                  const v4i (&w)[C::BPW][2],
                                                  const int (&bread)[C::NB],
                                                  int ones,
                                                  v16i (&acc)[C::BPW][2][C::NB],
                                                  int& tsum_part) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    v4i b[C::NB];
#pragma unroll
    for (int i = 0; i < C::NB; ++i)
      b[i] = *reinterpret_cast<const v4i*>(act + bread[i] + 16 * s);
#pragma unroll
    for (int bb = 0; bb < C::BPW; ++bb) {
      const v4i a0 = expand((uint32_t)w[bb][0][s]);
      const v4i a1 = expand((uint32_t)w[bb][1][s]);
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
        acc[bb][0][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            a0, b[i], acc[bb][0][i], 0, 0, 0);
        acc[bb][1][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            a1, b[i], acc[bb][1][i], 0, 0, 0);
      }
    }
    tsum_part = sdot4(b[0].x, ones, tsum_part);
    tsum_part = sdot4(b[0].y, ones, tsum_part);
    tsum_part = sdot4(b[0].z, ones, tsum_part);
    tsum_part = sdot4(b[0].w, ones, tsum_part);
  }
}

// Per-wave state of one workgroup tile.
template <class C>
struct TileState {
  const void* wbase[C::BPW];  // the wave's weight blocks
  int wbytes[C::BPW];
  const void* abase;  // the tile's activation rows
  int abytes;
  int av[C::kActDma];         // per-lane source offsets of the activation loads
  int aq[C::kActDma];         // their load indices q (uniform)
  int bread[C::NB];           // LDS offsets of the B operands
  int wread;                  // LDS offset (or source offset) of the A words
  int wave, lane, h, nfull;
  int c_begin;  // first chunk of the tile's reduction range
  v4i wreg[C::kRegW ? C::NS : 1][C::BPW][2];  // register ring of weights
  v16i acc[C::BPW][2][C::NB];
  int tsum_part;
  float sav[C::NB];  // activation scale of the lane's token in each tile
};

// Loads of stage st into ring slot S: activation loads, then the wave's two
// weight chunks (into LDS, or into the slot's registers).
template <class C, int S>
__device__ __forceinline__ void issue(TileState<C>& x, int st) {
  int8_t* act = act_slot<C, S>();
  const int c0 = x.c_begin + st * CPS;
#pragma unroll
  for (int r = 0; r < C::kActDma; ++r)
    load_lds16(x.abase, x.abytes, act + x.aq[r] * 1024, x.av[r] + c0 * 64);
  if constexpr (C::kRegW) {
    // the wait at the top of a stage counts the loads younger than the
    // stage's activation loads, so the scheduler must not move the weight
    // loads (plain loads, free to pass the direct-to-LDS ones) above them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < C::BPW; ++b) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<void*>(x.wbase[b]), 0, x.wbytes[b], kRsrcFlags);
      // streamed once: non-temporal
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2)
        x.wreg[S][b][r2] = __builtin_amdgcn_raw_buffer_load_b128(
            r, x.wread + c0 * 1024 + r2 * 512, 0, 2);
    }
  } else {
    int8_t* wts = wts_slot<C, S>();
#pragma unroll
    for (int j = 0; j < CPS; ++j)
      load_lds16(x.wbase[0], x.wbytes[0], wts + (x.wave * CPS + j) * 1024,
                 x.lane * 16 + (c0 + j) * 1024);
  }
}

// Loads younger than the activation loads of the stage in slot S, at its
// wait.  In the last, partial pass around the ring every stage issued is past
// the end: its weight loads into registers are never read, so the compiler
// drops them, and stage S finds S * kWLoads fewer younger loads than a full
// pass has (the count is exact then, and stricter than needed if they stay).
template <class C, int S, bool Last>
constexpr int younger() {
  return Last && C::kRegW ? C::kYounger - S * C::kWLoads : C::kYounger;
}

// Stage st from slot S; stage st + NS - 1 goes into slot S - 1 (mod NS),
// whose previous stage every wave finished before the barrier.
template <class C, int S, bool Last>
__device__ __forceinline__ void run_stage(TileState<C>& x, int st) {
  static_assert(younger<C, S, Last>() >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(younger<C, S, Last>()));
  __builtin_amdgcn_s_barrier();
  issue<C, (S + C::NS - 1) % C::NS>(x, st + C::NS - 1);
  // keep register-bound weight loads at the top of the stage: the scheduler
  // would otherwise sink them below the stage's math and shorten the
  // prefetch distance
  if constexpr (C::kRegW) __builtin_amdgcn_sched_barrier(0);
  if constexpr (C::kRegW)
    compute_stage_reg<C>(act_slot<C, S>(), x.wreg[S], x.bread,
                         (x.h == 0 || st < x.nfull) ? 0x01010101 : 0, x.acc,
                         x.tsum_part);
  else
    compute_stage<C>(act_slot<C, S>(), wts_slot<C, S>(), x.bread, x.wread,
                     st < x.nfull ? 0x01010101 : 0, x.acc[0], x.tsum_part);
}

// Slots S .. NS-1 of one pass around the ring, starting at stage st0; the
// Last (partial) pass runs only the stages below nst.
template <class C, int S, bool Last>
__device__ __forceinline__ void ring_pass(TileState<C>& x, int st0, int nst) {
  if constexpr (S < C::NS) {
    if (!Last || st0 + S < nst) run_stage<C, S, Last>(x, st0 + S);
    ring_pass<C, S + 1, Last>(x, st0, nst);
  }
}

// Loads of stages S .. NS-2 into their slots.  The scheduler may mix a
// stage's weight loads with the next stage's loads: that only adds loads
// younger than a stage's activation loads, so the waits stay sufficient.
template <class C, int S>
__device__ __forceinline__ void prologue(TileState<C>& x) {
  if constexpr (S < C::NS - 1) {
    issue<C, S>(x, S);
    prologue<C, S + 1>(x);
  }
}

// Direct stores of the wave's final sums (no staging): lane (h, i) writes
// its token's rows as four 16-byte pieces per register set.  Used for
// 32-token tiles holding at most kDirectTokens tokens: over the 2B-shaped
// decode set the two ways tie at 5 to 7 tokens, direct stores are ahead
// below that (90.0 against 93.4 us at 4), and the staged whole segments
// from 8 tokens on (95.5 against 99.2 us at 8, 102.6 against 108.5 at 16).
constexpr int kDirectTokens = 6;
template <class C>
__device__ __forceinline__ void store_direct(const Desc& d,
                                             const TileState<C>& x,
                                             v16i (&fin)[2][C::NB], int blk,
                                             int tok0) {
  const int lane = x.lane, h = x.h, li = lane & 31, wave = x.wave;
#pragma unroll
  for (int i = 0; i < C::NB; ++i) {
    const int tok = tok0 + 32 * ((i + wave) % C::NB) + li;
    if (tok >= d.m) continue;
    const float sa = x.sav[i];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int row = blk * 64 + 32 * r2 + 8 * g4 + 4 * h;
        v4i a, v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = fin[r2][i][4 * g4 + r];
          v[r] = __float_as_int(__fmul_rn(__fmul_rn((float)a[r], d.sw), sa));
        }
        store_row16<float, false>(d.y, d.n, tok, row,
                                  reinterpret_cast<const int8_t*>(&v));
        if (d.acc)
          store_row16<int32_t, false>(d.acc, d.n, tok, row,
                                      reinterpret_cast<const int8_t*>(&a));
      }
  }
}

// The staging region of a wave (TP tokens x kEpRow bytes) inside the ring's
// activation slots.
template <class C>
struct Staging {
  static constexpr int kPerSlot = C::kActSlot / kEpRow;  // tokens per slot
  // tokens per pass: 32 when two waves share a slot or a wave has one of
  // its own, else 16
  static constexpr int TP =
      C::kActSlot >= 2 * 32 * kEpRow ? 32 : (kPerSlot >= 32 ? 32 : 16);
  static_assert(TP * kEpRow <= C::kActSlot, "staging fits a slot");
  static_assert(C::kActSlot >= 2 * 32 * kEpRow || C::NS >= BLK,
                "one slot per wave");
};
template <class C>
__device__ __forceinline__ int8_t* staging(int wave) {
  if constexpr (C::kActSlot >= 2 * 32 * kEpRow) {
    int8_t* base = wave < 2 ? act_slot<C, 0>() : act_slot<C, 1>();
    return base + (wave & 1) * 32 * kEpRow;
  } else {
    switch (wave) {
      case 0: return act_slot<C, 0>();
      case 1: return act_slot<C, 1>();
      case 2: return act_slot<C, 2>();
      default: return act_slot<C, 3>();
    }
  }
}

// Writes the wave's final int32 sums fin (net of the activation sums) as y
// (and acc when requested) through the staging region.  fin[r2][i] holds
// rows 32 r2 + 8 (g / 4) + 4 h + g % 4 of token 32 ((i + wave) % NB) + li.
template <class C>
__device__ __forceinline__ void store_tile(const Desc& d, const TileState<C>& x,
                                           v16i (&fin)[2][C::NB], int blk,
                                           int tok0) {
  constexpr int NB = C::NB;
  constexpr int TP = Staging<C>::TP;
  if constexpr (NB == 1) {
    if (d.m - tok0 <= kDirectTokens) {  // few tokens: store directly
      store_direct<C>(d, x, fin, blk, tok0);
      return;
    }
  }
  const int lane = x.lane, h = x.h, li = lane & 31, wave = x.wave;
  int8_t* ep = staging<C>(wave);
  const int row = blk * 64 + 4 * (lane & 15);
#pragma unroll
  for (int pass_acc = 0; pass_acc < 2; ++pass_acc) {
    if (pass_acc == 1 && d.acc == nullptr) break;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int tl0 = 32 * ((i + wave) % NB);  // first token of this tile
      const float sa = x.sav[i];
#pragma unroll
      for (int p = 0; p < 32 / TP; ++p) {
        // lanes of tokens p TP .. p TP + TP - 1 write their rows
        if (li >= p * TP && li < (p + 1) * TP) {
          int8_t* w = ep + (li - p * TP) * kEpRow;
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              v4i v;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int a = fin[r2][i][4 * g4 + r];
                v[r] = pass_acc == 0
                           ? __float_as_int(
                                 __fmul_rn(__fmul_rn((float)a, d.sw), sa))
                           : a;
              }
              *reinterpret_cast<v4i*>(w + (32 * r2 + 8 * g4 + 4 * h) * 4) = v;
            }
        }
        // every lane stores 16 bytes of token p TP + 4 j + lane / 16
#pragma unroll
        for (int j = 0; j < TP / 4; ++j) {
          const int t = 4 * j + (lane >> 4);
          const int tk = tok0 + tl0 + p * TP + t;
          if (tk < d.m) {
            const int8_t* src = ep + t * kEpRow + 16 * (lane & 15);
            if (pass_acc == 0)
              store_row16<float, true>(d.y, d.n, tk, row, src);
            else
              store_row16<int32_t, true>(d.acc, d.n, tk, row, src);
          }
        }
      }
    }
  }
}

// Partial sums of a tile whose reduction is split over nsplit ranges: range
// ks stores its int32 partials (already net of its activation sums) in its
// own scratch region, in the accumulator layout [r2][tile][register][lane]
// so that each store covers 256 contiguous bytes, with device-scope stores
// that write through to the coherence point.  Once they are complete it
// counts its arrival with one device-scope atomic; the range that arrives
// last reads the other ranges' regions with device-scope loads, adds them
// to its own sums, clears the counter for the next launch and stores the
// outputs.  Integer addition is exact and order-free.
template <class C>
__device__ __forceinline__ void combine_split(const Desc& d, TileState<C>& x,
                                              v16i (&fin)[2][C::NB], int blk,
                                              int tt, int ks, int tok0,
                                              int32_t* sacc, int32_t* scnt) {
  constexpr int NB = C::NB;
  constexpr int64_t R = 64 * C::BM;  // ints per region
  const int lane = x.lane;
  const int64_t tile = (int64_t)blk * d.ntt + tt;
  const int64_t slot = d.slot0 + tile;
  int32_t* regions = sacc + (d.region0 + tile * d.nsplit) * R;
  int32_t* own = regions + ks * R;
#pragma unroll
  for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int g = 0; g < 16; ++g)
        __hip_atomic_store(own + ((r2 * NB + i) * 16 + g) * 64 + lane,
                           fin[r2][i][g], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  // the partials are at the coherence point before the arrival is counted
  __builtin_amdgcn_s_waitcnt(0);
  int arrived = 0;
  if (lane == 0) arrived = atomicAdd(scnt + slot, 1);
  arrived = __builtin_amdgcn_readfirstlane(arrived);
  if (arrived == d.nsplit - 1) {
    for (int r = 0; r < d.nsplit; ++r) {
      if (r == ks) continue;
      const int32_t* other = regions + r * R;
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int g = 0; g < 16; ++g)
            fin[r2][i][g] += __hip_atomic_load(
                other + ((r2 * NB + i) * 16 + g) * 64 + lane, __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) atomicExch(scnt + slot, 0);
    store_tile<C>(d, x, fin, blk, tok0);
  }
}

// One workgroup tile: weight rows [kRows rt, kRows rt + kRows) x tokens
// [BM tt, BM tt + BM), reduction over chunks [c_begin, c_end) (range ks of
// the problem's split).
template <class C>
__device__ __forceinline__ void run_tile(const Desc& d, int rt, int tt,
                                         int ks, int c_begin, int c_end,
                                         int32_t* sacc, int32_t* scnt) {
  constexpr int NB = C::NB;
  int* tsum = tsum_array<C>();
  TileState<C> x;
  const int tid = threadIdx.x;
  x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  x.lane = tid & 63;
  const int wave = x.wave;
  const int h = x.lane >> 5;
  const int li = x.lane & 31;
  const int k = d.k;
  const int nc = c_end - c_begin;
  const int nst = (nc + CPS - 1) / CPS;
  x.nfull = nc / CPS;  // full stages; an odd count (last range) adds one
  x.c_begin = c_begin;
  const int blk0 = (rt * BLK + wave) * C::BPW;  // the wave's first block
  const bool blk_ok = blk0 < d.nblk;            // wave-uniform

  // weight loads: each of the wave's blocks, 1 KiB per chunk, lane = 16-byte
  // row piece; a block past the problem's rows reads as zero
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    const bool ok = blk0 + b < d.nblk;
    x.wbase[b] = d.w + (size_t)(ok ? blk0 + b : 0) * 16 * (size_t)k;
    x.wbytes[b] = ok ? 16 * k : 0;
  }
  // activation loads: load q fills slot granules 64 q + lane, granule g of
  // the slot being byte 16 (g % 9) of token g / 9 (the ninth is padding and
  // gets a copy of the eighth; granules past the tile's tokens are out of
  // range).  Wave w issues loads q = w + 4 r.
  const int tok0 = tt * C::BM;
  x.abase = d.xq + (size_t)tok0 * k;
  x.abytes = min(C::BM, d.m - tok0) * k;
#pragma unroll
  for (int r = 0; r < C::kActDma; ++r) {
    const int q = min(wave + BLK * r, C::kActLoads - 1);
    x.aq[r] = q;
    const int g = q * 64 + x.lane;
    const int t = g / kRowGran;
    const int xg = min(g % kRowGran, kRowGran - 2);
    x.av[r] = t * k + xg * 16;
  }
  // matrix-core reads: B operand i is token 32 ((i + wave) % NB) + li,
  // inputs 64 j + 32 h + 16 s + [0, 16) of the stage
  x.h = h;
  if constexpr (C::kRegW) {
    // lane (h, li) takes chunk 2 p + h of rows li and 32 + li: B operands
    // from inputs 64 h + [0, 64) of the stage
#pragma unroll
    for (int i = 0; i < NB; ++i)
      x.bread[i] = (32 * ((i + wave) % NB) + li) * kRow + 64 * h;
    x.wread = h * 1024 + li * 16;
  } else {
    // lane (h, li) takes words 2h, 2h + 1 of each chunk of rows li, 32 + li
#pragma unroll
    for (int i = 0; i < NB; ++i)
      x.bread[i] = (32 * ((i + wave) % NB) + li) * kRow + 32 * h;
    x.wread = wave * CPS * 1024 + li * 16 + 8 * h;
  }
#pragma unroll
  for (int b = 0; b < C::BPW; ++b)
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
      for (int i = 0; i < NB; ++i) x.acc[b][r2][i] = v16i{0};
  x.tsum_part = 0;
  // the epilogue's activation scales, requested now so that the end of the
  // tile does not wait for them (older than every load of the ring, so the
  // ring's wait counts are unchanged)
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int tok = tok0 + 32 * ((i + wave) % NB) + li;
    x.sav[i] = tok < d.m ? *((gcfloat_ptr)d.sa + tok) : 0.0f;
  }

  // Prologue: stages 0 .. NS-2 in flight.  Every stage issues one more (past
  // the end they read out of range or unused rows and are never consumed),
  // so exactly NS-2 stages are younger than the one awaited.
  prologue<C, 0>(x);
  int st = 0;
  for (; st + C::NS <= nst; st += C::NS) ring_pass<C, 0, false>(x, st, nst);
  ring_pass<C, 0, true>(x, st, nst);
  // drain the loads issued past the end before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // activation sums of token tile `wave`: lanes li and li + 32 hold the two
  // input halves of token 32 wave + li
  const int ts = x.tsum_part + __shfl_xor(x.tsum_part, 32, 64);
  if (h == 0 && wave < NB) tsum[wave * 32 + li] = ts;
  __syncthreads();

  if (!blk_ok) return;
  int qs[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) qs[i] = tsum[32 * ((i + wave) % NB) + li];
  // every block unrolled with its own accumulators (a loop with an exit
  // would index them at run time and put them in scratch)
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    if (blk0 + b < d.nblk) {  // wave-uniform
      // sums net of the activation sums, in place
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int g = 0; g < 16; ++g) x.acc[b][r2][i][g] -= qs[i];
      if (d.nsplit > 1)
        combine_split<C>(d, x, x.acc[b], blk0 + b, tt, ks, tok0, sacc, scnt);
      else
        store_tile<C>(d, x, x.acc[b], blk0 + b, tok0);
    }
  }
}

template <class C>
__global__ __launch_bounds__(256, 2) void tiled_kernel(Desc d, int ntt) {
  const int u = blockIdx.x;
  // the division runs on the vector unit: copied to SGPRs (the compiler
  // drops a readfirstlane of a value it knows is uniform), the buffer
  // descriptors built from the tile indices need no per-lane loop
  int rt, tt;
  asm("s_mov_b32 %0, %1" : "=s"(rt) : "s"(u / ntt));
  asm("s_mov_b32 %0, %1" : "=s"(tt) : "s"(u % ntt));
  run_tile<C>(d, rt, tt, 0, 0, d.k >> 6, nullptr, nullptr);
}

// Unit sub-index: (row tile * ntt + token tile) * nsplit + range, row tiles
// of C::kRows rows; a unit of problem -1 is padding and does nothing.
template <class C>
__global__ __launch_bounds__(256, 2) void tiled_grouped_kernel(
    const Desc* __restrict__ descs, const Unit* __restrict__ units,
    int32_t* sacc, int32_t* scnt) {
  const Unit u = units[blockIdx.x];
  if (u.prob < 0) return;  // padding of an XCD-ordered plan
  const Desc d = descs[u.prob];
  const int ntt = (d.m + C::BM - 1) / C::BM;
  const int tile = u.sub / d.nsplit;
  const int ks = u.sub % d.nsplit;
  const int c_begin = ks * d.split_len;
  const int c_end = min(c_begin + d.split_len, d.k >> 6);
  run_tile<C>(d, tile / ntt, tile % ntt, ks, c_begin, c_end, sacc, scnt);
}

template <class C>
hipError_t launch_one(const Desc& d, hipStream_t s) {
  const int ntt = (d.m + C::BM - 1) / C::BM;
  const int64_t units = (int64_t)((d.n + C::kRows - 1) / C::kRows) * ntt;
  tiled_kernel<C><<<dim3((unsigned)units), dim3(256), 0, s>>>(d, ntt);
  return hipGetLastError();
}

template <class C>
hipError_t launch_group(const Desc* descs, const Unit* units, int64_t count,
                        int32_t* sacc, int32_t* scnt, hipStream_t s) {
  tiled_grouped_kernel<C><<<dim3((unsigned)count), dim3(256), 0, s>>>(
      descs, units, sacc, scnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(const Desc& d, hipStream_t s) {
  switch (token_tile(d.m)) {
    case 32: return launch_one<CfgS32>(d, s);
    case 64: return launch_one<CfgS64>(d, s);
    default: return launch_one<CfgP128>(d, s);
  }
}

hipError_t launch_tiled_grouped(const Desc* descs, const Unit* units,
                                int64_t count, int m, int32_t* sacc,
                                int32_t* scnt, hipStream_t s) {
  switch (token_tile(m)) {
    case 32: return launch_group<CfgS32>(descs, units, count, sacc, scnt, s);
    case 64: return launch_group<CfgS64>(descs, units, count, sacc, scnt, s);
    default: return launch_group<CfgP128>(descs, units, count, sacc, scnt, s);
  }
}

}  // namespace bt
