// Grouped ternary GEMV / very skinny GEMM (m <= 4) over many independent
// problems in one persistent launch: the decode step of a ternary model.
//
// The step is bound by HBM bandwidth: every packed weight is read once and
// used m <= 4 times ("1bit-systems" page, section "性能实测：92%的内存带宽
// 利用率": the ternary GEMV saturates memory; only reading fewer bytes makes
// it faster).  The kernel is therefore organised around the read stream:
//
//  * All problems' packed weights, in the 64-row-tiled layout, form one
//    logical stream of 1 KiB chunks (chunk = 64 rows x 64 inputs).  Inside a
//    problem, chunk L is at byte offset L * 1024, row block L / kc, input
//    chunk L % kc.
//  * The grid is persistent (a few workgroups per CU).  Wave w of W streams
//    chunks [w T / W, (w + 1) T / W) (W <= T): every wave reads the same
//    number of bytes, whatever the problem shapes.
//  * Lane l of a wave owns row 64 rb + l; for chunk L it loads 16 bytes with
//    one non-temporal 128-bit load (the wave reads 1 contiguous KiB); a wave
//    issues a group of D chunks, then consumes them, and the other resident
//    waves keep HBM busy meanwhile.
//  * The 64 activation bytes of a chunk are the same for every lane: scalar
//    loads bring them into SGPRs and v_dot4_i32_i8 takes them as an operand.
//    Each 2-bit field is masked in place (field j holds 4^j * code) and has
//    its own accumulator, combined with exact shifts at the end of a row
//    block.  Codes c = trit + 1 are used as they are; the finalising wave
//    subtracts the token's activation sum (sum (c - 1) q = sum c q - sum q;
//    bitnet.cpp CPU tutorial §1.1 for the sign-and-accumulate product).
//  * Finished row blocks are not stored at once: their sums wait in LDS
//    (up to 16 / m blocks per wave) and leave in one burst when the wave's
//    part of the problem is done, or when the staging area is full.  Writes
//    scattered through the read stream cost far more time than their bytes
//    (the memory has to turn the bus around for each of them).
//  * A row block cut by a wave-range boundary is shared by 2+ waves.  When
//    only two waves of one workgroup share it, their partial sums meet in
//    LDS at the end of the launch.  Otherwise each wave adds its partial
//    sums into 64-bit scratch slots that also count the block's chunks seen
//    so far (one device-scope atomic with return per row and token); the
//    lane that completes the count holds the total, writes the output and
//    clears the slot for the next launch.  The atomics are read-modify-writes
//    at the coherence point and cost far more than their bytes, so a full
//    grid runs 8-wave workgroups, one per CU, keeping 7 of every 8 cuts in
//    LDS.
#include "bt_internal.h"

namespace bt {

#ifdef BT_WAVE_TIMESTAMPS
// Timing build only (libbt_timing.so): each wave of a streaming launch
// writes the chip's 100 MHz real-time counter at fixed points of its work,
// and its hardware position, for the last launch.  Slots: 0 entry, 1 range
// and first problem known, 2 first weight group and activation sums
// arrived (fused plans: the first segment's rows quantized), 3 end of the
// last segment's loop, 4 hand-offs done, 5 after the workgroup barrier, 6
// exit, 7 segments streamed.
__device__ unsigned long long g_wave_ts[kTimedWaves * kTimedSlots];
__device__ unsigned int g_wave_hw[kTimedWaves * 2];
__device__ __forceinline__ void wave_stamp(int slot) {
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const unsigned long long t = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0 && w < kTimedWaves)
    g_wave_ts[w * kTimedSlots + slot] = t;
}
#define BT_STAMP(slot) wave_stamp(slot)
#else
#define BT_STAMP(slot) ((void)0)
#endif
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int* const_iptr;
typedef const __attribute__((address_space(4))) float* const_fptr;
typedef const __attribute__((address_space(4))) WaveStart* const_start_ptr;
typedef const __attribute__((address_space(1))) v4u* gv4u_ptr;
typedef __attribute__((address_space(1))) float* gfloat_ptr;
typedef __attribute__((address_space(1))) int32_t* gint_ptr;
typedef const __attribute__((address_space(1))) int* gcint_ptr;
typedef const __attribute__((address_space(1))) float* gcfloat_ptr;
typedef float v4f __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) v4f* gcfloat4_ptr;
typedef __attribute__((address_space(3))) int8_t* lds_i8_ptr;
typedef __attribute__((address_space(3))) uint32_t* lds_u32_ptr;
typedef const __attribute__((address_space(3))) v4u* lds_cv4u_ptr;

constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit words


constexpr int D = 4;  // chunks per load group
// load groups in flight per wave: with 8 waves per CU, 3 or 4 groups were no
// faster on the 2B and 8B decode sets (and 4 waves per CU with 2 to 4 groups
// 5-17 % slower, the dot products then lacking a second wave per SIMD to
// overlap with), although a bare read of 1 GiB with the same loads is
// fastest at 4 waves per CU and 3 or 4 groups
constexpr int G = 2;

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Sum over the 64 lanes, returned in a scalar register: DPP adds within each
// row of 16 lanes, then the four row totals are read out.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad 1032
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad 2301
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); // half mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Index of the last problem whose first chunk is <= pos (chunk0 ascending),
// with what a wave needs to start streaming it.  Every lane reads 4 entries
// per round, so up to 256 problems take a single memory round trip; in the
// first round each lane also reads its entries' weight and activation
// pointers and shape, so that the wave's first loads do not wait for a
// second, dependent descriptor read.
struct ProbStart {
  int p;
  bool have;  // the fields below are filled (the problem is among the first
              // 256)
  int kc, nblk;
  int64_t chunk0;
  const uint8_t* w;
  const void* x;  // int8 (xq) or, for fused plans, fp32 (xf) activations
};

// Lane l's 64-bit value (the readlane builtin moves 32 bits).
__device__ __forceinline__ int64_t read64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <bool FUSED>
__device__ __forceinline__ ProbStart find_problem(const Desc* descs,
                                                  const int64_t* chunk0,
                                                  int count, int64_t pos) {
  const int lane = threadIdx.x & 63;
  int p = 0;
  int64_t v[4];
  const uint8_t* wp[4];
  const void* xp[4];
  int kc[4], nb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = u * 64 + lane;
    const bool ok = i < count;
    const Desc& d = descs[ok ? i : 0];
    v[u] = ok ? chunk0[i] : INT64_MAX;
    wp[u] = d.w;
    xp[u] = FUSED ? (const void*)d.xf : (const void*)d.xq;
    kc[u] = d.kc;
    nb[u] = d.nblk;
  }
  bool more = true;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint64_t mask = __ballot(v[u] <= pos);
    p += __popcll(mask);
    more = more && mask == ~0ull;
  }
  ProbStart r;
  r.have = !more || count <= 256;
  for (int base = 256; more && base < count; base += 256) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * 64 + lane;
      v[u] = i < count ? chunk0[i] : INT64_MAX;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t mask = __ballot(v[u] <= pos);
      p += __popcll(mask);
      more = more && mask == ~0ull;
    }
  }
  r.p = __builtin_amdgcn_readfirstlane(p - 1);
  r.w = nullptr;
  r.x = nullptr;
  r.kc = r.nblk = 0;
  r.chunk0 = 0;
  if (r.have) {
    const int u = r.p >> 6, l = r.p & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j == u) {
        r.kc = __builtin_amdgcn_readlane(kc[j], l);
        r.nblk = __builtin_amdgcn_readlane(nb[j], l);
        r.chunk0 = read64(v[j], l);
        r.w = (const uint8_t*)read64((int64_t)wp[j], l);
        r.x = (const void*)read64((int64_t)xp[j], l);
      }
    }
  }
  return r;
}

template <int TOK>
struct Acc {
  int f[4][TOK];  // per 2-bit field j: sum of (4^j * code) * q
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < TOK; ++t) f[0][t] = f[1][t] = f[2][t] = f[3][t] = 0;
  }
  __device__ __forceinline__ int total(int t) const {
    return f[0][t] + (f[1][t] >> 2) + (f[2][t] >> 4) + f[3][t];
  }
  // Empty volatile asm that reads and writes every accumulator: the dot
  // products issued so far complete before any later volatile asm, which
  // keeps each pair of chunks' work in program order.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int t = 0; t < TOK; ++t)
      asm volatile("" : "+v"(f[0][t]), "+v"(f[1][t]), "+v"(f[2][t]),
                   "+v"(f[3][t]));
  }
};

// A run of cnt <= D consecutive chunks inside row block rb, starting at input
// chunk c (problem-local chunk index rb * kc + c).  All 32-bit and uniform.
struct Group {
  int rb, c, cnt;
  // Re-assert that the fields are wave-uniform (scalar registers); without
  // it the compiler keeps the loop-carried copies in VGPRs, where its
  // bookkeeping would overwrite registers of loads still in flight.
  __device__ __forceinline__ void uniform() {
    rb = __builtin_amdgcn_readfirstlane(rb);
    c = __builtin_amdgcn_readfirstlane(c);
    cnt = __builtin_amdgcn_readfirstlane(cnt);
  }
};

// FUSED: the problem gives fp32 activations; each wave quantizes the rows it
// needs into LDS (exactly as the quantization kernel does) and reads the
// int8 values from there instead of through scalar loads.
// CHAIN (persistent chained launch, FUSED only): the outputs are read later
// in the same launch by waves on other XCDs, so they are stored at agent
// scope (written through to the device's coherence point); the inputs are
// read after an agent-scope acquire that drops stale cached copies.
template <int TOK, bool FUSED, bool CHAIN = false>
struct Stream {
  // problem
  const uint8_t* w;  // the problem's packed weights
  const int8_t* xq;
  gcfloat_ptr xf;    // FUSED: fp32 activations [TOK, k]
  gcfloat_ptr gain;  // FUSED with RMSNorm: per-feature gain [k], else null
  float eps;
  lds_i8_ptr xl;     // FUSED: this wave's LDS copy of the quantized rows
  const_fptr sa;     // scalar loads: a vector load would wait behind the
                     // weight loads in flight
  gfloat_ptr y;
  gint_ptr accout;
  float sw;
  int n, k, kc, blk0;
  int64_t chunk0;
  // wave range (global chunks) and grid
  int64_t lo, hi;
  // the neighbouring waves' ranges [prev_lo, lo) and [hi, next_hi), and
  // whether they belong to this workgroup
  int64_t prev_lo, next_hi;
  bool prev_in_wg, next_in_wg;
  // cut blocks shared with a neighbour of this workgroup and no one else:
  // their partial sums meet in LDS after the stream (see stream_kernel)
  bool head_local, tail_local;
#ifdef BT_WAVE_TIMESTAMPS
  bool ts_first = true;
  int ts_segments = 0;
#endif
  int tail_rb_local;
  int head_keep[TOK], tail_keep[TOK];
  int32_t* sacc;
  int qsum[TOK];
  float sav[TOK];    // the tokens' activation scales (read once per problem)
  // LDS staging of finished row blocks: kOut blocks of TOK rows of 64 sums;
  // ocnt blocks are staged, the first of them is row block orb0, and the
  // rest follow it (a segment finishes its whole blocks in order).
  static constexpr int kOut = 16 / TOK;
  int* obuf;
  int ocnt, orb0;

  // Next group after g in a segment ending at problem-local chunk s1.
  __device__ __forceinline__ Group next(Group g, int s1) const {
    Group r;
    r.rb = g.rb;
    r.c = g.c + g.cnt;
    if (r.c == kc) {
      r.c = 0;
      ++r.rb;
    }
    r.cnt = max(0, min(min(D, kc - r.c), s1 - (r.rb * kc + r.c)));
    r.uniform();
    return r;
  }

  // Loads are unconditional: they go through a buffer resource that spans
  // exactly the group's g.cnt chunks, so slots past g.cnt (and every slot of
  // the empty group after the last) read as zero without touching memory.
  // Streamed once: non-temporal.
  __device__ __forceinline__ void load_group(v4u (&buf)[D], Group g) const {
    const int start = g.rb * kc + g.c;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (size_t)start * 1024), 0, g.cnt * 1024, kRsrcFlags);
    const int lane16 = (threadIdx.x & 63) * 16;
#pragma unroll
    for (int j = 0; j < D; ++j)
      buf[j] = __builtin_bit_cast(
          v4u, __builtin_amdgcn_raw_buffer_load_b128(r, lane16 + j * 1024, 0, 2));
  }

  // The 64 activation bytes of input chunk c for every token (SGPRs).
  struct QChunk {
    int v[TOK][16];
  };
  __device__ __forceinline__ void load_q(QChunk& qc, int c, int pin) const {
    if constexpr (FUSED) {
      // every lane reads the same 16 bytes: LDS broadcasts them
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        const lds_cv4u_ptr q = (lds_cv4u_ptr)(xl + t * k + c * 64 + pin);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4u v = q[i];
          qc.v[t][4 * i + 0] = (int)v.x;
          qc.v[t][4 * i + 1] = (int)v.y;
          qc.v[t][4 * i + 2] = (int)v.z;
          qc.v[t][4 * i + 3] = (int)v.w;
        }
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const_iptr q = (const_iptr)(xq + (size_t)t * k + (size_t)c * 64 + pin);
#pragma unroll
      for (int i = 0; i < 16; ++i) qc.v[t][i] = q[i];
    }
  }

  // Chunk wv with activations qc.  A chunk past the group's end reads as
  // zero bytes: codes 0, which contribute nothing.
  __device__ __forceinline__ void dot_chunk(const v4u& wv, const QChunk& qc,
                                            Acc<TOK>& a) const {
    const uint32_t m0 = 0x03030303u, m1 = 0x0C0C0C0Cu, m2 = 0x30303030u;
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const int e0 = (int)(words[ww] & m0);
        const int e1 = (int)(words[ww] & m1);
        const int e2 = (int)(words[ww] & m2);
        const int e3 = (int)((words[ww] >> 6) & m0);
        a.f[0][t] = sdot4(e0, qc.v[t][4 * ww + 0], a.f[0][t]);
        a.f[1][t] = sdot4(e1, qc.v[t][4 * ww + 1], a.f[1][t]);
        a.f[2][t] = sdot4(e2, qc.v[t][4 * ww + 2], a.f[2][t]);
        a.f[3][t] = sdot4(e3, qc.v[t][4 * ww + 3], a.f[3][t]);
      }
    }
  }

  // All D chunks are consumed unconditionally (chunks past g.cnt read as
  // zero and use a clamped activation chunk), so the compiler keeps every
  // load of the group ahead of the first use instead of sinking loads into
  // branches.  Chunks go in runs of P: the run's activations are requested
  // together (one wait per run), and an opaque zero on their addresses plus
  // an accumulator pin after the run keep at most P chunks' activations
  // (16 SGPRs per chunk and token) live.
  static constexpr int P = TOK == 1 ? 2 : 1;
  __device__ __forceinline__ void consume(const v4u (&buf)[D], Group g,
                                          Acc<TOK>& a) const {
#pragma unroll
    for (int j = 0; j < D; j += P) {
      int pin;
      asm volatile("s_mov_b32 %0, 0" : "=s"(pin));
      QChunk q[P];
#pragma unroll
      for (int r = 0; r < P; ++r) load_q(q[r], min(g.c + j + r, kc - 1), pin);
#pragma unroll
      for (int r = 0; r < P; ++r)
        dot_chunk(buf[j + r], q[r], a);
      a.pin();
    }
  }

  // Writes the staged row blocks and empties the staging area.
  __device__ __forceinline__ void flush() {
    const int lane = threadIdx.x & 63;
    for (int i = 0; i < ocnt; ++i) {
#pragma unroll
      for (int t = 0; t < TOK; ++t)
        write_one(orb0 + i, t, obuf[(i * TOK + t) * 64 + lane]);
    }
    orb0 += ocnt;
    ocnt = 0;
  }

  // One output of row block rb, token t (lane = row).
  __device__ __forceinline__ void write_one(int rb, int t, int sum) {
    const int row = rb * 64 + (threadIdx.x & 63);
    if (row >= n) return;
    const int acc = sum - qsum[t];
    const size_t o = (size_t)t * n + row;
    const float yv = __fmul_rn(__fmul_rn((float)acc, sw), sav[t]);
    if constexpr (CHAIN) {
      if (accout != nullptr)
        __hip_atomic_store((int32_t*)accout + o, acc, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store((float*)y + o, yv, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (accout != nullptr) accout[o] = acc;
      y[o] = yv;
    }
  }

  // This wave holds only part of row block rb (partial sums in sum[]).  Each
  // (row, token) of the block has a 64-bit scratch slot holding
  // (chunks << 32) + partial total: one atomic add with return of
  // (c << 32) + partial adds this wave's share, c chunks of the block's kc.
  // The lane that sees the chunk count reach kc holds the total (the partial
  // totals stay below 2^31 in magnitude, so the two fields decode exactly);
  // it writes the output and clears the slot for the next launch.  Counting
  // chunks rather than contributors makes the hand-off independent of how
  // the stream was cut.  Integer addition is exact and order-free; no lane
  // waits for another.  A wave has at most two such blocks (the first and
  // the last of its range).  Blocks shared only by two waves of one
  // workgroup do not come here: they meet in LDS (see stream_kernel).
  struct HandOff {
    uint64_t ret[TOK];  // what the atomics returned (slot before the add)
    int64_t delta[TOK];
    int rb;
  };

  __device__ __forceinline__ unsigned long long* slot_of(int rb) const {
    return reinterpret_cast<unsigned long long*>(sacc) +
           ((int64_t)blk0 + rb) * (TOK * 64) + (threadIdx.x & 63);
  }

  __device__ __forceinline__ void hand_off(HandOff& h, int rb,
                                           const int (&sum)[TOK],
                                           int chunks) const {
    unsigned long long* sp = slot_of(rb);
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      h.delta[t] = ((int64_t)chunks << 32) + (int64_t)sum[t];
      h.ret[t] = atomicAdd(sp + t * 64, (unsigned long long)h.delta[t]);
    }
    h.rb = rb;
  }

  __device__ __forceinline__ void settle(const HandOff& h) {
    unsigned long long* sp = slot_of(h.rb);
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const int64_t now = (int64_t)h.ret[t] + h.delta[t];
      const int64_t chunks = (now + ((int64_t)1 << 31)) >> 32;
      if (chunks == kc) {
        write_one(h.rb, t, (int)(now - ((int64_t)kc << 32)));
        atomicExch(sp + t * 64, 0ull);  // at the coherence point too
      }
    }
  }

  // Sum of each token's activations (needed when finishing rows).  The
  // first kActPer 16-byte pieces per lane and token are loaded before the
  // segment's first weight groups (issue_act) and summed after those groups
  // have been issued (finish_act): the sum then waits only for its own
  // loads, which are older, and the weight stream keeps going.  Rows longer
  // than kActPer KiB (rare: k > 8192 at m = 1) load the rest afterwards.
  static constexpr int kActPer = TOK == 1 ? 8 : (TOK == 2 ? 7 : (TOK == 3 ? 4 : 3));
  struct ActPre {
    v4u v[TOK][kActPer];
  };
  __device__ __forceinline__ void issue_act(ActPre& p) const {
    const int lane = threadIdx.x & 63;
    const int n16 = k >> 4;  // 16-byte pieces per token row
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const gv4u_ptr q16 = (gv4u_ptr)(xq + (size_t)t * k);
#pragma unroll
      for (int u = 0; u < kActPer; ++u)  // clamped, unconditional
        p.v[t][u] = q16[min(u * 64 + lane, n16 - 1)];
    }
  }
  __device__ __forceinline__ void finish_act(const ActPre& p) {
    const int lane = threadIdx.x & 63;
    const int n16 = k >> 4;
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      int s = 0;
#pragma unroll
      for (int u = 0; u < kActPer; ++u) {
        const int ones = u * 64 + lane < n16 ? 0x01010101 : 0;
        s = sdot4((int)p.v[t][u].x, ones, s);
        s = sdot4((int)p.v[t][u].y, ones, s);
        s = sdot4((int)p.v[t][u].z, ones, s);
        s = sdot4((int)p.v[t][u].w, ones, s);
      }
      const gv4u_ptr q16 = (gv4u_ptr)(xq + (size_t)t * k);
      for (int i0 = kActPer * 64; i0 < n16; i0 += 4 * 64) {
        v4u v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * 64 + lane;
          v[u] = i < n16 ? q16[i] : v4u{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s = sdot4((int)v[u].x, 0x01010101, s);
          s = sdot4((int)v[u].y, 0x01010101, s);
          s = sdot4((int)v[u].z, 0x01010101, s);
          s = sdot4((int)v[u].w, 0x01010101, s);
        }
      }
      qsum[t] = wave_sum(s);
    }
  }

  // FUSED: quantize the problem's TOK activation rows into this wave's LDS
  // area with the quantization kernel's arithmetic (quant_scale, quant4),
  // taking each row's activation sum and scale on the way.  The row is read
  // in batches of kBatch float4 per lane whose loads are all issued before
  // any is used (one round trip per batch); a row of at most one batch
  // stays in registers between the absmax and the quantization, longer rows
  // are read a second time (from cache).
  static constexpr int kBatch = 8;
  // float4 i of an activation row (in a chained launch, read after the
  // barrier's acquire, which dropped stale cached copies)
  __device__ __forceinline__ v4f ldx(gcfloat4_ptr xr, int i) const {
    return xr[i];
  }
  __device__ __forceinline__ void load_batch(float4 (&v)[kBatch],
                                             gcfloat4_ptr xr, int b0,
                                             int n4) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // clamped: repeats change no maximum
      const v4f f = ldx(xr, min(b0 + u * 64 + lane, n4 - 1));
      v[u] = make_float4(f.x, f.y, f.z, f.w);
    }
  }
  __device__ __forceinline__ void quant_batch(const float4 (&v)[kBatch],
                                              lds_u32_ptr dst, int b0, int n4,
                                              float inv, int& s) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = b0 + u * 64 + lane;
      if (i < n4) {
        const uint32_t q = quant4(v[u], inv);
        dst[i] = q;
        s = sdot4((int)q, 0x01010101, s);
      }
    }
  }
  // FUSED with RMSNorm: the same three passes as the standalone kernel
  // (sum of squares in the fixed order of sumsq4, normalized absmax,
  // rounding), so both give the same bytes.
  __device__ __forceinline__ void norm_rows() {
    const int lane = threadIdx.x & 63;
    const int n4 = k >> 2;
    const gcfloat4_ptr gr = (gcfloat4_ptr)gain;
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const gcfloat4_ptr xr = (gcfloat4_ptr)(xf + (size_t)t * k);
      const lds_u32_ptr dst = (lds_u32_ptr)(xl + t * k);
      float4 v[kBatch];
      double ss = 0.0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = u * 64 + lane;
        const v4f f = i < n4 ? ldx(xr, i) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
        v[u] = make_float4(f.x, f.y, f.z, f.w);
        if (i < n4) ss = sumsq4(ss, v[u]);
      }
      for (int b0 = 64 * kBatch; b0 < n4; b0 += 64 * kBatch)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = b0 + u * 64 + lane;
          if (i < n4) {
            const v4f f = ldx(xr, i);
            ss = sumsq4(ss, make_float4(f.x, f.y, f.z, f.w));
          }
        }
      const float r = rms_scale(wave_sum_f64(ss), k, eps);
      float amax = 0.0f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = u * 64 + lane;
        if (i < n4) {
          const v4f gv = gr[i];
          v[u] = rms_apply(v[u], r, make_float4(gv.x, gv.y, gv.z, gv.w));
          amax = fmaxf(amax, absmax4(v[u]));
        }
      }
      for (int b0 = 64 * kBatch; b0 < n4; b0 += 64 * kBatch)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = b0 + u * 64 + lane;
          if (i < n4) {
            const v4f f = ldx(xr, i), gv = gr[i];
            amax = fmaxf(amax, absmax4(rms_apply(
                make_float4(f.x, f.y, f.z, f.w), r,
                make_float4(gv.x, gv.y, gv.z, gv.w))));
          }
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const QScale qs = quant_scale(amax);
      int s = 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = u * 64 + lane;
        if (i < n4) {
          const uint32_t q = quant4(v[u], qs.inv);
          dst[i] = q;
          s = sdot4((int)q, 0x01010101, s);
        }
      }
      for (int b0 = 64 * kBatch; b0 < n4; b0 += 64 * kBatch)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = b0 + u * 64 + lane;
          if (i < n4) {
            const v4f f = ldx(xr, i), gv = gr[i];
            const uint32_t q = quant4(
                rms_apply(make_float4(f.x, f.y, f.z, f.w), r,
                          make_float4(gv.x, gv.y, gv.z, gv.w)),
                qs.inv);
            dst[i] = q;
            s = sdot4((int)q, 0x01010101, s);
          }
        }
      qsum[t] = wave_sum(s);
      sav[t] = qs.sa;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  __device__ __forceinline__ void quantize_rows() {
    if (gain != nullptr) {
      norm_rows();
      return;
    }
    const int n4 = k >> 2;
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const gcfloat4_ptr xr = (gcfloat4_ptr)(xf + (size_t)t * k);
      const lds_u32_ptr dst = (lds_u32_ptr)(xl + t * k);
      float4 v[kBatch];
      float amax = 0.0f;
      load_batch(v, xr, 0, n4);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) amax = fmaxf(amax, absmax4(v[u]));
      for (int b0 = 64 * kBatch; b0 < n4; b0 += 64 * kBatch) {
        float4 w[kBatch];
        load_batch(w, xr, b0, n4);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) amax = fmaxf(amax, absmax4(w[u]));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const QScale qs = quant_scale(amax);
      int s = 0;
      quant_batch(v, dst, 0, n4, qs.inv, s);  // the first batch is still here
      for (int b0 = 64 * kBatch; b0 < n4; b0 += 64 * kBatch) {
        float4 w[kBatch];
        load_batch(w, xr, b0, n4);
        quant_batch(w, dst, b0, n4, qs.inv, s);
      }
      qsum[t] = wave_sum(s);
      sav[t] = qs.sa;
    }
    // the rows are read back by other lanes of this wave only: LDS keeps a
    // wave's operations in order; the clobber keeps the compiler from
    // moving the reads above the writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // State of a segment between the issue of its first weight groups and the
  // rest of its work (a persistent launch issues them before it waits for
  // the segment's inputs).
  struct Seg {
    int s0, s1, head_rb;
    bool head_cut;
    Group g, pg;  // the group consumed next and the last group issued
    v4u ring[G][D];
  };

  // First groups of chunks [s0, s1) of the current problem in flight.
  __device__ __forceinline__ void seg_issue(Seg& sg, int s0, int s1) const {
    s0 = __builtin_amdgcn_readfirstlane(s0);
    s1 = __builtin_amdgcn_readfirstlane(s1);
    sg.s0 = s0;
    sg.s1 = s1;
    sg.head_rb = s0 / kc;
    sg.head_cut = s0 != sg.head_rb * kc;  // first block starts early
    sg.g.rb = sg.head_rb;
    sg.g.c = s0 - sg.head_rb * kc;
    sg.g.cnt = min(min(D, kc - sg.g.c), s1 - s0);
    sg.g.uniform();
    sg.pg = next(sg.g, s1);
    load_group(sg.ring[0], sg.g);
#pragma unroll
    for (int i = 1; i < G; ++i) {
      if (i > 1) sg.pg = next(sg.pg, s1);
      load_group(sg.ring[i], sg.pg);
    }
  }

  // FUSED: the rest of a segment whose first groups are in flight: quantize
  // the rows, then stream and hand off.
  __device__ __forceinline__ void seg_run(Seg& sg) {
    int head_sum[TOK];
#pragma unroll
    for (int t = 0; t < TOK; ++t) head_sum[t] = 0;
    Acc<TOK> a;
    a.zero();
    ocnt = 0;
    orb0 = sg.head_rb + (sg.head_cut ? 1 : 0);  // first block finished whole
    quantize_rows();
#ifdef BT_WAVE_TIMESTAMPS
    if (ts_first) BT_STAMP(2);
    ts_first = false;
    ++ts_segments;
#endif
    stream_rest(sg.ring, sg.g, sg.pg, sg.s0, sg.s1, sg.head_rb, sg.head_cut,
                head_sum, a);
  }

  // Stream chunks [s0, s1) of the current problem (problem-local indices) in
  // groups of up to D chunks, G groups in flight: while one group is
  // consumed, the next G - 1 are in flight.  Every load is unconditional
  // (range-checked), so the wait before each group is a fixed count (the
  // other groups' loads); the loop's only other memory operations are LDS
  // writes and the occasional burst of a full staging area.  A row block cut
  // by the range (at most the first and the last) keeps its partial sums in
  // registers; their hand-off happens after the loop.
  __device__ __forceinline__ void segment(int s0, int s1) {
    if constexpr (FUSED) {
      Seg sg;
      seg_issue(sg, s0, s1);
      seg_run(sg);
      return;
    }
    s0 = __builtin_amdgcn_readfirstlane(s0);
    s1 = __builtin_amdgcn_readfirstlane(s1);
    const int head_rb = s0 / kc;
    const bool head_cut = s0 != head_rb * kc;  // first block starts early
    int head_sum[TOK];
#pragma unroll
    for (int t = 0; t < TOK; ++t) head_sum[t] = 0;
    Group g;
    g.rb = head_rb;
    g.c = s0 - head_rb * kc;
    g.cnt = min(min(D, kc - g.c), s1 - s0);
    g.uniform();
    Group pg = next(g, s1);
    Acc<TOK> a;
    a.zero();
    ocnt = 0;
    orb0 = head_rb + (head_cut ? 1 : 0);  // the first block finished whole
    // G groups in flight: ring slot i holds the i-th group from g on, and pg
    // is the last group issued
    v4u ring[G][D];
    load_group(ring[0], g);
    ActPre pre;
    issue_act(pre);
#pragma unroll
    for (int i = 1; i < G; ++i) {
      if (i > 1) pg = next(pg, s1);
      load_group(ring[i], pg);
    }
    finish_act(pre);
#ifdef BT_WAVE_TIMESTAMPS
    if (ts_first) BT_STAMP(2);
    ts_first = false;
    ++ts_segments;
#endif
#pragma unroll
    for (int t = 0; t < TOK; ++t) sav[t] = sa[t];
    stream_rest(ring, g, pg, s0, s1, head_rb, head_cut, head_sum, a);
  }

  // The loop of a segment and its hand-offs.
  __device__ __forceinline__ void stream_rest(v4u (&ring)[G][D], Group g,
                                              Group pg, int s0, int s1,
                                              int head_rb, bool head_cut,
                                              int (&head_sum)[TOK],
                                              Acc<TOK>& a) {
    bool more = true;
    while (more) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        g.uniform();
        pg.uniform();
        consume(ring[i], g, a);
        group_end(g, head_rb, head_cut, head_sum, a);
        pg = next(pg, s1);
        load_group(ring[i], pg);
        g = next(g, s1);
        if (g.cnt == 0) {
          more = false;
          break;
        }
      }
    }
    BT_STAMP(3);
    // The staged blocks go first; then both hand-offs are issued, and only
    // then are the atomics' results looked at.  The cut head block's sums
    // were stashed only if it also ended here; otherwise it is the last
    // block and still sits in the accumulators.
    flush();
    bool head_off = head_cut && (head_rb + 1) * kc <= s1;
    bool tail_off = s1 % kc != 0;  // the range ends inside a block
    int tail_sum[TOK];
#pragma unroll
    for (int t = 0; t < TOK; ++t) tail_sum[t] = a.total(t);
    const int tail_rb = (s1 - 1) / kc;
    // A cut block that only this wave and its neighbour in the workgroup
    // share (it starts inside the neighbour's range or this one's and ends
    // inside the other) skips the atomics: both waves reach the same
    // decision from the same ranges.
    if (head_off && prev_in_wg && chunk0 + (int64_t)head_rb * kc >= prev_lo) {
      head_local = true;
#pragma unroll
      for (int t = 0; t < TOK; ++t) head_keep[t] = head_sum[t];
      head_off = false;
    }
    if (tail_off && next_in_wg && tail_rb * kc >= s0 &&
        chunk0 + (int64_t)(tail_rb + 1) * kc <= next_hi) {
      tail_local = true;
      tail_rb_local = tail_rb;
#pragma unroll
      for (int t = 0; t < TOK; ++t) tail_keep[t] = tail_sum[t];
      tail_off = false;
    }
    // Only blocks that are cut take the atomics; both are issued before
    // either result is looked at, so the round trips overlap.
    HandOff hh, ht;
    if (head_off) hand_off(hh, head_rb, head_sum, (head_rb + 1) * kc - s0);
    if (tail_off) hand_off(ht, tail_rb, tail_sum, s1 - max(tail_rb * kc, s0));
    if (head_off) settle(hh);
    if (tail_off) settle(ht);
  }

  // After each group: a group that ends a row block either stages the block
  // (whole in this wave's range) or, for the cut head block, keeps its sums
  // for the hand-off after the loop.
  __device__ __forceinline__ void group_end(Group g, int head_rb,
                                            bool head_cut,
                                            int (&head_sum)[TOK],
                                            Acc<TOK>& a) {
    const bool end = g.c + g.cnt == kc;
    const bool head = end && head_cut && g.rb == head_rb;
    int sum[TOK];
#pragma unroll
    for (int t = 0; t < TOK; ++t) sum[t] = a.total(t);
    if (head) {
#pragma unroll
      for (int t = 0; t < TOK; ++t) head_sum[t] = sum[t];
    }
    if (end && !head) {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int t = 0; t < TOK; ++t) obuf[(ocnt * TOK + t) * 64 + lane] = sum[t];
      if (++ocnt == kOut) flush();
    }
    if (end) a.zero();
  }
};

// Chunks [lo, hi) of the concatenated stream, problem by problem.
// `start`: the wave's entry of the plan's start table (problem p holds chunk
// lo), or null: then the wave searches the problems' first chunks.
template <int TOK, bool FUSED>
__device__ __forceinline__ void stream_range(Stream<TOK, FUSED>& st,
                                             const Desc* __restrict__ descs,
                                             const int64_t* __restrict__ chunk0s,
                                             const WaveStart* start, int count,
                                             int64_t lo, int64_t hi) {
  if (lo >= hi) return;
  st.lo = lo;
  st.hi = hi;
  ProbStart ps;
  if (start) {
    // scalar loads of the entry (a wave-uniform address)
    const const_start_ptr e = (const_start_ptr)start;
    ps.p = e->p;
    ps.have = true;
    ps.kc = e->kc;
    ps.nblk = e->nblk;
    ps.chunk0 = e->chunk0;
    ps.w = e->w;
    ps.x = e->x;
  } else {
    ps = find_problem<FUSED>(descs, chunk0s, count, lo);
  }
  BT_STAMP(1);
  int p = ps.p;
  int64_t pos = lo;
  bool first = ps.have;
  while (pos < hi && p < count) {
    const Desc& d = descs[p];
    int64_t chunks;
    if (first) {
      // start from the lookup's fields; the rest of the descriptor is read
      // alongside the first loads and used only after them
      st.w = ps.w;
      if constexpr (FUSED)
        st.xf = (gcfloat_ptr)ps.x;
      else
        st.xq = (const int8_t*)ps.x;
      st.kc = ps.kc;
      st.k = ps.kc * 64;
      st.chunk0 = ps.chunk0;
      chunks = (int64_t)ps.nblk * ps.kc;
      first = false;
    } else {
      st.w = d.w;
      st.xq = d.xq;
      st.xf = (gcfloat_ptr)d.xf;
      st.kc = d.kc;
      st.k = d.k;
      st.chunk0 = d.chunk0;
      chunks = (int64_t)d.nblk * d.kc;
    }
    if constexpr (FUSED) {
      st.gain = (gcfloat_ptr)d.g;
      st.eps = d.eps;
    }
    st.sa = (const_fptr)d.sa;
    st.y = (gfloat_ptr)d.y;
    st.accout = (gint_ptr)d.acc;
    st.sw = d.sw;
    st.n = d.n;
    st.blk0 = d.blk0;
    const int64_t s0 = pos - st.chunk0;
    const int64_t s1 = min(chunks, hi - st.chunk0);
    st.segment((int)s0, (int)s1);
    pos = st.chunk0 + s1;
    ++p;
  }
  BT_STAMP(4);
}

// Wave wv of W streams chunks [wv T / W, (wv + 1) T / W) of the T chunks.
// Waves of one launch finish several microseconds apart (whole XCDs run
// slower or faster from launch to launch), but the launch is bound by the
// total bytes over the aggregate HBM rate: a wave that ends early leaves its
// share of the bandwidth to the others.  Handing out the stream's tail
// dynamically (from shared counters, or through a claiming wave per
// workgroup with work stealing across XCDs) evened out the ends and made
// the launch slower, not faster.
//
// WPW waves per workgroup: 8 for a full grid with int8 activations (one
// workgroup per CU, the same 8 waves per CU as two of 4), so that 7 of every
// 8 range boundaries fall inside a workgroup and their cut blocks meet in
// LDS; 4 for smaller plans, which then spread over more CUs, and when the
// launch quantizes (the LDS copies of the rows, 16 KiB per wave, leave room
// for no more).
template <int TOK, bool FUSED, int WPW>
__global__ __launch_bounds__(64 * WPW) void stream_kernel(
    const Desc* __restrict__ descs, const int64_t* __restrict__ chunk0s,
    const WaveStart* __restrict__ starts, int count, int64_t total,
    int32_t* sacc) {
  static_assert(WPW == 4 || (WPW == 8 && !FUSED), "workgroup shape");
  // With fewer chunks than waves, only the first `total` waves take part.
  const int64_t W = min((int64_t)gridDim.x * WPW, total);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wv = (int64_t)blockIdx.x * WPW + wave;
  BT_STAMP(0);
#ifdef BT_WAVE_TIMESTAMPS
  if ((threadIdx.x & 63) == 0 && wv < kTimedWaves) {
    g_wave_hw[wv * 2] = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
    g_wave_hw[wv * 2 + 1] =
        __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));
  }
#endif
  Stream<TOK, FUSED> st;
  __shared__ int obuf_all[WPW][16 * 64];
  st.obuf = obuf_all[wave];
  // FUSED: each wave's quantized activation rows (m * k <= BT_FUSED_MAX_MK)
  __shared__ v4u xl_all[WPW][FUSED ? BT_FUSED_MAX_MK / 16 : 1];
  st.xl = (lds_i8_ptr)xl_all[wave];
  st.sacc = sacc;
  st.head_local = false;
  st.tail_local = false;
  if (wv < W) {
    // the neighbours share this workgroup only if they take part too
    st.prev_in_wg = wave > 0;
    st.next_in_wg = wave < WPW - 1 && wv + 1 < W;
    int64_t lo, hi;
    if (starts) {  // the plan's entry for this wave (scalar loads)
      const const_start_ptr e = (const_start_ptr)(starts + wv);
      lo = e->lo;
      hi = e->hi;
      st.prev_lo = e->prev_lo;
      st.next_hi = e->next_hi;
    } else {
      lo = wv * total / W;
      hi = (wv + 1) * total / W;
      st.prev_lo = wv > 0 ? (wv - 1) * total / W : 0;
      st.next_hi = wv + 1 < W ? (wv + 2) * total / W : total;
    }
    stream_range(st, descs, chunk0s, starts ? starts + wv : nullptr, count,
                 lo, hi);
  }
  // Cut blocks shared by two waves of this workgroup only: the wave that
  // holds the block's last chunks leaves its partial sums in its (now
  // empty) staging area, and the wave that holds the first chunks adds them
  // to its own and writes the outputs.  Every wave of the workgroup reaches
  // this barrier, including those without a range.
  const int lane = threadIdx.x & 63;
  if (st.head_local) {
#pragma unroll
    for (int t = 0; t < TOK; ++t) st.obuf[t * 64 + lane] = st.head_keep[t];
  }
  __syncthreads();
  BT_STAMP(5);
  if (st.tail_local) {
    const int* other = obuf_all[wave + 1];
#pragma unroll
    for (int t = 0; t < TOK; ++t)
      st.write_one(st.tail_rb_local, t, st.tail_keep[t] + other[t * 64 + lane]);
  }
  BT_STAMP(6);
#ifdef BT_WAVE_TIMESTAMPS
  if (lane == 0 && wv < kTimedWaves)
    g_wave_ts[wv * kTimedSlots + 7] = st.ts_segments;
#endif
}

// ---------------------------------------------------------------------------
// Persistent chained decode: the phases of one token (each a fused plan whose
// fp32 input is an output of an earlier phase) in one cooperative launch,
// with a grid-wide barrier between phases.  A wave's range of a phase is
// split in two: range_begin finds the first problem and issues the first
// groups of its weights (which depend on nothing computed in the launch), so
// it runs before the barrier that precedes the phase; range_run quantizes
// the input and does the rest after it.

struct RangeCursor {
  int p;         // problem after the first segment
  int64_t pos;   // first chunk after the first segment
  bool active;   // the range is not empty
};

template <int TOK, bool CHAIN>
__device__ __forceinline__ void take_problem(Stream<TOK, true, CHAIN>& st,
                                             const Desc& d) {
  st.gain = (gcfloat_ptr)d.g;
  st.eps = d.eps;
  st.sa = (const_fptr)d.sa;
  st.y = (gfloat_ptr)d.y;
  st.accout = (gint_ptr)d.acc;
  st.sw = d.sw;
  st.n = d.n;
  st.blk0 = d.blk0;
}

template <int TOK, bool CHAIN>
__device__ __forceinline__ void range_begin(
    Stream<TOK, true, CHAIN>& st, typename Stream<TOK, true, CHAIN>::Seg& sg,
    RangeCursor& rc, const Desc* __restrict__ descs,
    const int64_t* __restrict__ chunk0s, int count, int64_t lo, int64_t hi) {
  rc.active = lo < hi;
  if (!rc.active) return;
  st.lo = lo;
  st.hi = hi;
  const ProbStart ps = find_problem<true>(descs, chunk0s, count, lo);
  const Desc& d = descs[ps.p];
  int64_t chunks;
  if (ps.have) {
    st.w = ps.w;
    st.xf = (gcfloat_ptr)ps.x;
    st.kc = ps.kc;
    st.k = ps.kc * 64;
    st.chunk0 = ps.chunk0;
    chunks = (int64_t)ps.nblk * ps.kc;
  } else {
    st.w = d.w;
    st.xf = (gcfloat_ptr)d.xf;
    st.kc = d.kc;
    st.k = d.k;
    st.chunk0 = d.chunk0;
    chunks = (int64_t)d.nblk * d.kc;
  }
  take_problem(st, d);
  const int64_t s0 = lo - st.chunk0;
  const int64_t s1 = min(chunks, hi - st.chunk0);
  st.seg_issue(sg, (int)s0, (int)s1);
  rc.p = ps.p + 1;
  rc.pos = st.chunk0 + s1;
}

template <int TOK, bool CHAIN>
__device__ __forceinline__ void range_run(
    Stream<TOK, true, CHAIN>& st, typename Stream<TOK, true, CHAIN>::Seg& sg,
    const RangeCursor& rc, const Desc* __restrict__ descs, int count) {
  if (!rc.active) return;
  st.seg_run(sg);
  int p = rc.p;
  int64_t pos = rc.pos;
  while (pos < st.hi && p < count) {
    const Desc& d = descs[p];
    st.w = d.w;
    st.xf = (gcfloat_ptr)d.xf;
    st.kc = d.kc;
    st.k = d.k;
    st.chunk0 = d.chunk0;
    take_problem(st, d);
    const int64_t chunks = (int64_t)d.nblk * d.kc;
    const int64_t s0 = pos - st.chunk0;
    const int64_t s1 = min(chunks, st.hi - st.chunk0);
    st.segment((int)s0, (int)s1);
    pos = st.chunk0 + s1;
    ++p;
  }
}

// Grid-wide barrier between phases (all workgroups resident: cooperative
// launch).  Every wave first waits for its own memory operations (its
// outputs are agent-scope stores, so they are then at the coherence point);
// after a workgroup barrier its first thread stores the phase number into
// the workgroup's arrival word.  Workgroup 0 watches every arrival word and
// then stores the phase number into the release word, which the first
// thread of every workgroup watches.  (Every workgroup watching every
// arrival word instead, without the release word, was slower: 1.62 against
// 1.38 ms per token of the 2B chained decode.)  All words are read and
// written at agent scope.  Every wait is bounded by the real-time clock: a
// workgroup that gives up sets the error word, every waiter also stops when
// it sees it, and the launch then ends with its outputs invalid.
constexpr uint64_t kChainTimeoutTicks = 50000000;  // 0.5 s at 100 MHz

__device__ __forceinline__ bool grid_barrier(uint32_t* sync, uint32_t target,
                                             int* ok_flag) {
  uint32_t* arrive = sync;
  uint32_t* gen = sync + kChainMaxWg;
  uint32_t* err = sync + kChainMaxWg + 1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0)
      __hip_atomic_store(arrive + blockIdx.x, target, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0) {
      while (true) {
        bool ok = true;
        for (int i = lane; i < (int)gridDim.x; i += 64)
          ok = ok && __hip_atomic_load(arrive + i, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) >= target;
        if (__all(ok)) break;
        if (__hip_atomic_load(err, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT) != 0)
          break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kChainTimeoutTicks) {
          if (lane == 0)
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0)
        __hip_atomic_store(gen, target, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else if (lane == 0) {
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) < target &&
             __hip_atomic_load(err, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == 0) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kChainTimeoutTicks) {
          __hip_atomic_store(err, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (lane == 0)
      *ok_flag = __hip_atomic_load(err, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == 0;
    // acquire: drop the XCD's L2 and this CU's L1 copies of lines that
    // other XCDs wrote in the phase just ended (the next phase's input),
    // so that the loads after the barrier fetch them afresh
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  return *ok_flag != 0;  // one value for the whole workgroup
}

// One token's phases.  A phase of T chunks is streamed by
// W = min(waves, max(1, T / 4)) waves (at least four chunks each, as the
// launched plans have), in equal ranges, exactly as stream_kernel does.
template <int TOK>
__global__ __launch_bounds__(256) void chain_kernel(
    const ChainPhase* __restrict__ phases, int nphase, uint32_t* sync) {
  constexpr int WPW = 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * WPW + wave;
  Stream<TOK, true, true> st;
  __shared__ int obuf_all[WPW][16 * 64];
  __shared__ v4u xl_all[WPW][BT_FUSED_MAX_MK / 16];
  __shared__ int ok_flag;
  st.obuf = obuf_all[wave];
  st.xl = (lds_i8_ptr)xl_all[wave];
  typename Stream<TOK, true, true>::Seg sg;
  RangeCursor rc;
  auto begin = [&](int ph) {
    const ChainPhase P = phases[ph];
    const int64_t total = P.total;
    const int64_t W = min((int64_t)gridDim.x * WPW, max((int64_t)1, total / 4));
    st.sacc = P.sacc;
    st.head_local = false;
    st.tail_local = false;
    rc.active = false;
    if (wv < W) {
      st.prev_lo = wv > 0 ? (wv - 1) * total / W : 0;
      st.next_hi = wv + 1 < W ? (wv + 2) * total / W : total;
      st.prev_in_wg = wave > 0;
      st.next_in_wg = wave < WPW - 1 && wv + 1 < W;
      range_begin(st, sg, rc, P.descs, P.chunk0, P.count, wv * total / W,
                  (wv + 1) * total / W);
    }
  };
  begin(0);
  for (int ph = 0; ph < nphase; ++ph) {
    range_run(st, sg, rc, phases[ph].descs, phases[ph].count);
    // cut blocks shared by two waves of this workgroup only (as in
    // stream_kernel)
    if (st.head_local) {
#pragma unroll
      for (int t = 0; t < TOK; ++t) st.obuf[t * 64 + lane] = st.head_keep[t];
    }
    __syncthreads();
    if (st.tail_local) {
      const int* other = obuf_all[wave + 1];
#pragma unroll
      for (int t = 0; t < TOK; ++t)
        st.write_one(st.tail_rb_local, t,
                     st.tail_keep[t] + other[t * 64 + lane]);
    }
    if (ph + 1 == nphase) break;
    begin(ph + 1);
    if (!grid_barrier(sync, (uint32_t)(ph + 1), &ok_flag)) return;
  }
}

}  // namespace

hipError_t launch_chain(const ChainPhase* phases, int nphase, int m,
                        uint32_t* sync, int workgroups, hipStream_t s) {
  void* args[] = {(void*)&phases, (void*)&nphase, (void*)&sync};
  const void* f;
  switch (m) {
    case 1: f = (const void*)chain_kernel<1>; break;
    case 2: f = (const void*)chain_kernel<2>; break;
    case 3: f = (const void*)chain_kernel<3>; break;
    case 4: f = (const void*)chain_kernel<4>; break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchCooperativeKernel(f, dim3((unsigned)workgroups), dim3(256),
                                    args, 0, s);
}

// `workgroups` counts 4-wave workgroups; with WPW = 8 the same waves are
// regrouped in half as many.
template <bool FUSED, int WPW>
hipError_t launch_stream(const Desc* descs, const int64_t* chunk0,
                         const WaveStart* starts, int32_t count,
                         int64_t total_chunks, int m, int32_t* sacc,
                         int workgroups, hipStream_t s) {
  const dim3 grid((unsigned)((workgroups * 4 + WPW - 1) / WPW)), block(64 * WPW);
  switch (m) {
    case 1: stream_kernel<1, FUSED, WPW><<<grid, block, 0, s>>>(descs, chunk0, starts, count, total_chunks, sacc); break;
    case 2: stream_kernel<2, FUSED, WPW><<<grid, block, 0, s>>>(descs, chunk0, starts, count, total_chunks, sacc); break;
    case 3: stream_kernel<3, FUSED, WPW><<<grid, block, 0, s>>>(descs, chunk0, starts, count, total_chunks, sacc); break;
    case 4: stream_kernel<4, FUSED, WPW><<<grid, block, 0, s>>>(descs, chunk0, starts, count, total_chunks, sacc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_grouped(const Desc* descs, const int64_t* chunk0,
                                 const WaveStart* starts, int32_t count,
                                 int64_t total_chunks, int m, int32_t* sacc,
                                 int workgroups, bool fused, bool full,
                                 hipStream_t s) {
  if (fused)
    return launch_stream<true, 4>(descs, chunk0, starts, count, total_chunks,
                                  m, sacc, workgroups, s);
  // a full grid runs one workgroup per CU (all of the CU's waves)
  return full ? launch_stream<false, 4 * kStreamWgPerCu>(
                    descs, chunk0, starts, count, total_chunks, m, sacc,
                    workgroups, s)
              : launch_stream<false, 4>(descs, chunk0, starts, count,
                                        total_chunks, m, sacc, workgroups, s);
}

}  // namespace bt

#ifdef BT_WAVE_TIMESTAMPS
extern "C" int32_t bt_wave_timestamps(uint64_t* ts, uint32_t* hw) {
  if (!ts || !hw) return BT_E_NULL;
  if (hipMemcpyFromSymbol(ts, HIP_SYMBOL(bt::g_wave_ts),
                          sizeof(bt::g_wave_ts)) != hipSuccess ||
      hipMemcpyFromSymbol(hw, HIP_SYMBOL(bt::g_wave_hw),
                          sizeof(bt::g_wave_hw)) != hipSuccess)
    return BT_E_HIP;
  return BT_OK;
}
#endif
