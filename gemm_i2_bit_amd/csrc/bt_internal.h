// Internal declarations shared by the library's HIP translation units.
// Device code targets gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bt.h"

namespace bt {

// One problem as the kernels see it (the grouped plan stores an array of
// these in device memory; single calls pass one by value).
struct alignas(16) Desc {
  const uint8_t* w;   // packed weights, 64-row-tiled layout
  const int8_t* xq;   // int8 activations [m, k]
  const float* sa;    // activation scales [m]
  float* y;           // fp32 outputs [m, n]
  int32_t* acc;       // int32 accumulators [m, n] or nullptr
  float sw;           // weight scale
  int32_t n, k, m;
  int32_t nblk;       // 64-row blocks = ceil(n / 64)
  int32_t ntt;        // token tiles of the matrix-core kernels
  // grouped streaming path: position of this problem in the concatenated
  // stream of 1 KiB chunks, and its first row block in the scratch area
  int64_t chunk0;
  int32_t blk0;
  int32_t kc;         // k / 64 = chunks per row block
  // matrix-core kinds: the reduction of every tile is split into nsplit
  // ranges of split_len chunks (even; the last range may be shorter); with
  // nsplit > 1, 64-row block b and token tile t count the arrivals of their
  // ranges in counter slot0 + b * ntt + t, and range r leaves its partial
  // sums in scratch region region0 + (b * ntt + t) * nsplit + r
  int32_t nsplit;
  int32_t split_len;
  int32_t slot0;
  int32_t region0;
  // fused-quantization plans: fp32 activations [m, k] (xq and sa are null)
  const float* xf;
  // fused plans with RMSNorm: per-feature gain [k] (null: no norm) and eps
  const float* g;
  float eps;
  int32_t pad_;
};
static_assert(sizeof(Desc) == 128, "Desc is 128 bytes");

// One work unit of a grouped launch: problem index and a sub-index whose
// meaning depends on the kernel: for the matrix-core kinds,
// (row tile * ntt + token tile) * nsplit + reduction range (row tiles of
// tile_rows(token tile) rows).  Problem -1
// marks padding that keeps an XCD-ordered unit list aligned.
struct Unit {
  int32_t prob;
  int32_t sub;
};

// Where one wave of a streaming launch starts: the wave's range of the
// concatenated chunk stream (wave w of W streams chunks [w T / W,
// (w + 1) T / W) of the T chunks), its neighbours' range ends, and the
// problem that holds its first chunk with what the wave needs to issue its
// first weight loads.  One entry is one cache line, read with scalar loads;
// without the table every wave divides for its bounds and searches the
// problems' first chunks, every lane gathering descriptors, at the start of
// the launch: a median 2.5 us of the 2B set's M=1 launch went by before a
// wave's first weight load.
struct WaveStart {
  const uint8_t* w;  // packed weights of problem p
  const void* x;     // int8 (xq) or, for fused plans, fp32 (xf) activations
  int64_t chunk0;    // first chunk of problem p in the stream
  int64_t lo, hi;    // the wave's chunks [lo, hi)
  int32_t p;
  int32_t kc;        // chunks per row block of problem p
  int32_t nblk;      // row blocks of problem p
  int32_t pad0_;
  int64_t prev_lo;   // first chunk of the previous wave (0 for wave 0)
  int64_t next_hi;   // end of the next wave's range (T for the last wave)
  int64_t pad_[7];
};
static_assert(sizeof(WaveStart) == 128, "WaveStart is 128 bytes");

// Host-side header at the start of a grouped plan image.  Layout:
//   PlanHeader | Desc[count] | int64 chunk0[count] | WaveStart[start_waves] |
//   Unit[units] | int32 scratch_acc[...] | int32 scratch_cnt[...]
// The streaming kind has units = 0, one slot of m * 64 int64 (arrival count
// in the high half, partial total in the low half) per row block, and no
// counters.  Its start table is written for the wave count of a launch on
// the device that was current when the plan was built (start_waves = 0 if
// none was); a launch with another wave count searches instead.
// The matrix-core kinds have, for the problems whose reduction is split, one
// region of 64 * token_tile ints per (row block, token tile, range) and one
// counter per (row block, token tile); none otherwise.
struct PlanHeader {
  uint32_t magic;
  int32_t count;
  int32_t m;
  int32_t kind;        // kKindDot4, kKindMfma or kKindPrefill
  int64_t units;
  int64_t desc_off;    // byte offset of Desc[count]
  int64_t chunk_off;   // byte offset of int64 chunk0[count]
  int64_t unit_off;    // byte offset of Unit[units]
  int64_t sacc_off;    // byte offset of the int32 partial sums
  int64_t scnt_off;    // byte offset of the int32 arrival counters
  int64_t bytes;       // total image size
  int64_t total_chunks;
  int64_t blocks;      // row blocks over all problems
  int64_t fused;       // 1: the problems give fp32 activations (Desc::xf)
  int64_t start_off;   // byte offset of WaveStart[start_waves]
  int64_t start_waves; // waves the start table is written for (0: none)
  int64_t pad[2];
};
static_assert(sizeof(PlanHeader) == 128, "PlanHeader is 128 bytes");

constexpr uint32_t kPlanMagic = 0x31475442u;  // "BTG1"
constexpr int kKindDot4 = 0;     // m <= 4: packed dot products
constexpr int kKindMfma = 1;     // 4 < m < kPrefillMinM: matrix-core tiles of
                                 // 32 or 64 tokens (weight-stream bound)
constexpr int kKindPrefill = 2;  // m >= kPrefillMinM: 128-token tiles
constexpr int kDot4MaxM = 4;
constexpr int kPrefillMinM = 65;

inline int plan_kind(int64_t m) {
  return m <= kDot4MaxM ? kKindDot4
                        : (m < kPrefillMinM ? kKindMfma : kKindPrefill);
}
// Kind of a grouped plan.  From 2 tokens on, the packed dot products of a
// large plan are bound by the vector ALUs (4 dot products per 16 inputs and
// token) rather than by the weight stream, and the matrix cores are faster
// over a 521 MB decode set: 87 against 96-103 us at m = 2, 93 against
// 124-136 us at m = 3, 98 against 142-158 us at m = 4.  Smaller plans stay
// faster on the dot products, whose launch starts streaming sooner (one
// 17 MB layer at m = 4; 87 MB at m = 2).  Plans that quantize their own
// activations always stream.
constexpr int64_t kSkinnyMfmaChunks = 32768;  // 32 MiB of packed weights
constexpr int64_t kPairMfmaChunks = 131072;   // 128 MiB, for m = 2
inline int group_kind(int64_t m, int64_t total_chunks, bool fused) {
  if (fused || m <= 1) return plan_kind(m);
  if (m <= kDot4MaxM) {
    const int64_t from = m == 2 ? kPairMfmaChunks : kSkinnyMfmaChunks;
    return total_chunks >= from ? kKindMfma : kKindDot4;
  }
  return plan_kind(m);
}
// tokens per workgroup tile of the matrix-core kernels
inline int token_tile(int64_t m) { return m <= 32 ? 32 : (m <= 64 ? 64 : 128); }
// weight rows per workgroup tile for a token tile: 64-token tiles give each
// of the 4 waves two 64-row blocks, the others one
constexpr int tile_rows(int token_tile) { return token_tile == 64 ? 512 : 256; }
// work units (tile_rows x token-tile workgroups) of one problem for the
// matrix-core kinds, before any split of the reduction
inline int64_t kind_units(int kind, int64_t n, int64_t m) {
  if (kind == kKindDot4) return 0;
  const int bm = token_tile(m);
  const int rows = tile_rows(bm);
  return (n + rows - 1) / rows * ((m + bm - 1) / bm);
}
// int32 entries of one split-reduction scratch region (64 rows x token tile)
inline int64_t split_region_ints(int64_t m) { return 64 * token_tile(m); }
#ifndef BT_STREAM_WG_PER_CU
#define BT_STREAM_WG_PER_CU 2
#endif
constexpr int kStreamWgPerCu = BT_STREAM_WG_PER_CU;  // persistent grid: WGs/CU
// Workgroups of 4 waves in a streaming launch over total_chunks on `cus`
// compute units: a persistent grid, but at least a group of 4 chunks per
// wave (a wave's set-up and hand-offs cost about what streaming a few chunks
// does, so small plans, one phase of a chained decode, run on fewer, fuller
// waves).  The kernel streams with min(4 * workgroups, total_chunks) waves.
inline int64_t stream_workgroups(int64_t total_chunks, int cus) {
  const int64_t full = (int64_t)cus * kStreamWgPerCu;
  const int64_t need = (total_chunks + 15) / 16;
  return full < need ? full : need;
}
inline int64_t stream_waves(int64_t total_chunks, int cus) {
  const int64_t w = 4 * stream_workgroups(total_chunks, cus);
  return w < total_chunks ? w : total_chunks;
}

// Timing build (BT_WAVE_TIMESTAMPS): waves recorded per launch and
// timestamp slots per wave.
constexpr int kTimedWaves = 4096;
constexpr int kTimedSlots = 8;

// Launchers (host code in the kernels' translation units).
hipError_t launch_pack(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                       int32_t* n_invalid, hipStream_t s);
hipError_t launch_quant(const float* x, int64_t m, int64_t k, int8_t* xq,
                        float* sa, hipStream_t s);
constexpr int kMaxQuantJobs = BT_MAX_QUANT_JOBS;
hipError_t launch_quant_many(const bt_quant_job* jobs, int32_t count,
                             hipStream_t s);
// Waves per 64-row block of the single-problem kernels: enough for about
// 2048 waves in all (8 per CU) when the matrix has few row blocks, at least
// 4 chunks of 64 inputs per wave, and 4, 8 or 16 waves.
inline int row_block_waves(int64_t nblk, int kc) {
  int w = 4;
  while (w < 16 && nblk * w < 2048 && kc >= 4 * (2 * w)) w *= 2;
  return w;
}
hipError_t launch_dot4(const Desc& d, hipStream_t s);
hipError_t launch_lut(const Desc& d, hipStream_t s);  // m = 1 only
// full: the grid fills every CU (workgroups == CUs * kStreamWgPerCu)
// starts: the plan's start table for this launch's wave count, or null
hipError_t launch_stream_grouped(const Desc* descs, const int64_t* chunk0,
                                 const WaveStart* starts, int32_t count,
                                 int64_t total_chunks, int m, int32_t* sacc,
                                 int workgroups, bool fused, bool full,
                                 hipStream_t s);

// One phase of a persistent chained launch: a fused plan's descriptors,
// chunk offsets and scratch slots in device memory.
struct ChainPhase {
  const Desc* descs;
  const int64_t* chunk0;
  int32_t* sacc;
  int64_t total;  // chunks of the phase
  int32_t count;  // problems of the phase
  int32_t pad_;
};
static_assert(sizeof(ChainPhase) == 40, "ChainPhase is 40 bytes");
// Sync words of a chained launch: an arrival word per workgroup (at most
// kChainMaxWg), the release word, the error word.
constexpr int kChainMaxWg = 1024;
constexpr int kChainSyncWords = kChainMaxWg + 64;
hipError_t launch_chain(const ChainPhase* phases, int nphase, int m,
                        uint32_t* sync, int workgroups, hipStream_t s);

// A token row's scales from its absmax: a = max(amax, 1e-5), one correctly
// rounded 127 / a for the products and s_a = a / 127 for the rescale.
struct QScale {
  float inv, sa;
};
__device__ __forceinline__ QScale quant_scale(float amax) {
  const float a = fmaxf(amax, 1e-5f);
  return QScale{__fdiv_rn(127.0f, a), __fdiv_rn(a, 127.0f)};
}

// Quantizes four activations with a row's 127 / a (fp32 product, round half
// to even, clamp +-127) and packs them as 4 int8 in a little-endian word.
// Shared by the quantization kernel and the fused streaming kernel so that
// both produce the same bytes.
__device__ __forceinline__ uint32_t quant4(const float4& v, float inv) {
  const float e[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed4 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r = rintf(__fmul_rn(e[j], inv));  // round half to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    packed4 |= ((uint32_t)(int32_t)r & 0xffu) << (8 * j);
  }
  return packed4;
}
// five-trits-per-byte comparison format (gemv_b3.hip)
int64_t b3_packed_bytes(int64_t n, int64_t k);
hipError_t launch_pack_b3(const int8_t* t, int64_t n, int64_t k,
                          uint8_t* packed, int32_t* n_invalid, hipStream_t s);
hipError_t launch_b3(const Desc& d, hipStream_t s);  // m = 1 only
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                             int waves, int wpw, int groups, hipStream_t s);
hipError_t launch_mix_probe(const void* buf, int64_t bytes, void* out,
                            int64_t out_bytes, int burst, uint32_t* sink,
                            int waves, int wpw, int groups, hipStream_t s);
// RMSNorm before the quantization.  A row's sum of squares is taken by one
// wave, in one fixed order, by every kernel that normalizes: lane l adds the
// squares of float4 i = l, l + 64, l + 128, ... in increasing i (x, y, z, w
// within each), in double (each square is exact), and the lanes combine by
// an xor butterfly over offsets 32, 16, ..., 1 (every lane ends with the
// same sum).  So the standalone and the fused kernels give identical bits.
__device__ __forceinline__ double sumsq4(double s, const float4& v) {
  s += (double)v.x * (double)v.x;
  s += (double)v.y * (double)v.y;
  s += (double)v.z * (double)v.z;
  s += (double)v.w * (double)v.w;
  return s;
}
__device__ __forceinline__ double wave_sum_f64(double s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}
// r = 1 / sqrt(ss / k + eps) in double, rounded once to fp32
__device__ __forceinline__ float rms_scale(double ss, int64_t k, float eps) {
  return (float)(1.0 / sqrt(ss / (double)k + (double)eps));
}
// h = (x * r) * g, two fp32 products
__device__ __forceinline__ float4 rms_apply(const float4& x, float r,
                                            const float4& g) {
  return make_float4(__fmul_rn(__fmul_rn(x.x, r), g.x),
                     __fmul_rn(__fmul_rn(x.y, r), g.y),
                     __fmul_rn(__fmul_rn(x.z, r), g.z),
                     __fmul_rn(__fmul_rn(x.w, r), g.w));
}
__device__ __forceinline__ float absmax4(const float4& v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}
hipError_t launch_norm_quant(const float* x, const float* g, int64_t m,
                             int64_t k, float eps, int8_t* xq, float* sa,
                             float* h, hipStream_t s);

hipError_t launch_tiled(const Desc& d, hipStream_t s);
hipError_t launch_tiled_grouped(const Desc* descs, const Unit* units,
                                int64_t count, int m, int32_t* sacc,
                                int32_t* scnt, hipStream_t s);

}  // namespace bt
