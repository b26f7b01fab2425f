/*
 * bt.h: C ABI of the W1.58A8 ternary GEMV/GEMM library for AMD MI355X
 * (CDNA4, gfx950).
 *
 * What is computed (readings of the pages are stated where they are silent):
 *  - Weights are ternary, one of -1, 0, +1 ("1bit-systems：在AMD Strix Halo上
 *    实现纯Rust本地三值权重LLM推理", section "三值量化：1.58-bit的魔法";
 *    bitnet.cpp CPU tutorial at m.qwbw.cn, §1.1), stored 2 bits each (same
 *    tutorial §1.1; the 2-bit format is named I2_S in "BitNet 1 位 LLM 独立推理
 *    引擎：位串行 GEMM 内核与 LUT 优化工程实践", conversion paragraph), with one
 *    fp32 scale s_w per tensor (the absmean of the conversion step, tutorial
 *    §3.2).
 *  - Activations are quantized to int8, one scale per token ("BitNet-rs：
 *    Rust实现的高效1比特大语言模型推理引擎", section "技术实现细节").
 *  - The product of a ternary weight and an activation is the activation, its
 *    negation or nothing; products are accumulated exactly in int32 (tutorial
 *    §1.1), then rescaled: y = ((float)acc * s_w) * s_a[token].
 *
 * Shapes: weights W are [n, k] (n outputs, k inputs), activations [m, k]
 * (m tokens), outputs [m, n].  All tensors are row-major and contiguous.
 *
 * Memory and ownership.  Every tensor pointer is a DEVICE pointer; the caller
 * allocates and owns every buffer.  The library allocates no memory, keeps no
 * per-call state and never synchronizes: each call checks its arguments on
 * the host, enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 * stream) and returns.  Calls on different streams are independent.
 *
 * Errors.  Argument checks run on the host before any HIP call and return a
 * negative status; a failed launch returns BT_E_HIP.  Bad data is reported
 * without a status: see bt_pack_i2s (invalid trits) and bt_quant_act
 * (non-finite inputs give unspecified results).
 */
#ifndef BT_H
#define BT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BT_OK 0
#define BT_E_NULL (-1)  /* a required pointer is NULL */
#define BT_E_SHAPE (-2) /* n, m or k out of range, k % 64 != 0, size mismatch */
#define BT_E_ALIGN (-3) /* a pointer is not aligned as documented */
#define BT_E_ARG (-4)   /* s_w negative or not finite, bad plan, bad count */
#define BT_E_HIP (-5)   /* the HIP runtime reported an error */
#define BT_E_ARCH (-6)  /* the current device is not gfx950 */

#define BT_MAX_K 65536         /* keeps |acc| <= 127 k < 2^24: (float)acc exact */
#define BT_MAX_N (1 << 28)
#define BT_MAX_M (1 << 24)

/* Short text for a status code (static storage). */
const char* bt_status_str(int32_t status);

/* Size in bytes of a packed [n, k] ternary tensor: ceil(n / 64) * 64 * k / 4.
 * Returns BT_E_SHAPE for n < 1, k < 64, k % 64 != 0, k > BT_MAX_K or
 * n > BT_MAX_N.
 *
 * Packed layout (this library's format; the pages name 2-bit storage and
 * I2_S but print no layout).  Code c = trit + 1: 0 -> -1, 1 -> 0, 2 -> +1;
 * code 3 is invalid.  Rows are padded to a multiple of 64 with code 1.
 * Row block b = r / 64 occupies bytes [b * 16 k, (b + 1) * 16 k).  Inside a
 * block, the 16-byte chunk holding inputs [64 c, 64 c + 64) of row r sits at
 * offset c * 1024 + (r % 64) * 16.  Inside a chunk, weight k is in byte
 * 4 ((k % 64) / 16) + (k % 4), at bits [2 ((k % 16) / 4), +2).  So a wave of
 * 64 lanes reads one contiguous KiB per chunk, one row per lane, and shifting
 * a 32-bit word right by 2 j and masking with 0x03030303 yields the codes of
 * 4 consecutive inputs, aligned with one 32-bit word of int8 activations. */
int64_t bt_packed_bytes(int64_t n, int64_t k);

/* Pack ternary weights.
 *  t         int8 [n, k] trits in {-1, 0, 1}, device, 16-byte aligned.
 *  packed    bt_packed_bytes(n, k) bytes, device, 16-byte aligned; written
 *            entirely (padding rows included).
 *  n_invalid nullable device int32: incremented by the number of entries of
 *            t outside {-1, 0, 1} (the caller zeroes it first).  Their packed
 *            fields hold code 3 and products over them are unspecified.
 * Offline step (conversion time); not on the per-token path. */
int32_t bt_pack_i2s(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                    int32_t* n_invalid, void* stream);

/* Per-token absmax int8 quantization of fp32 activations x [m, k].
 * For each row: amax = max |x|; a = max(amax, 1e-5f); inv = 127.0f / a
 * (correctly rounded); x_q = clamp(round_half_even(x * inv), -127, 127) with
 * an fp32 product; s_a = a / 127.0f (correctly rounded).
 *  x    fp32 [m, k], device, 16-byte aligned.
 *  x_q  int8 [m, k], device, 16-byte aligned.
 *  s_a  fp32 [m], device, 4-byte aligned.
 * Requires 1 <= m <= BT_MAX_M and the k rules of bt_packed_bytes.
 * Non-finite x gives unspecified x_q and s_a. */
int32_t bt_quant_act(const float* x, int64_t m, int64_t k, int8_t* x_q,
                     float* s_a, void* stream);

/* Several independent quantizations in one launch, each exactly
 * bt_quant_act(job.x, job.m, job.k, job.x_q, job.s_a): the per-token step of
 * a decode pass whose projections read activation matrices of different
 * widths.  jobs is a HOST array of 1 <= count <= BT_MAX_QUANT_JOBS entries,
 * read during the call only; each job obeys the rules of bt_quant_act, and
 * the total number of rows is at most BT_MAX_M.  Jobs must not overlap in
 * memory. */
#define BT_MAX_QUANT_JOBS 16
typedef struct bt_quant_job {
  const float* x;   /* fp32 [m, k], device, 16-byte aligned */
  int8_t* x_q;      /* int8 [m, k], device, 16-byte aligned */
  float* s_a;       /* fp32 [m], device, 4-byte aligned */
  int64_t m;
  int64_t k;
} bt_quant_job;
int32_t bt_quant_act_many(const bt_quant_job* jobs, int32_t count,
                          void* stream);

/* Ternary matrix-vector product (one token): bt_gemm with m = 1. */
int32_t bt_gemv(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                const int8_t* x_q, const float* s_a, float* y, int32_t* acc,
                void* stream);

/* The same product as bt_gemv (same arguments, rules and results, bit for
 * bit), computed with lookup tables instead of dot products: the table
 * method of the CPU kernels in "BitNet 1 位 LLM 独立推理引擎：位串行 GEMM 内核
 * 与 LUT 优化工程实践" (body: TL1 turns two weights into a 4-bit index into
 * precomputed tables of their ternary combinations).  Kept for comparison
 * only: on gfx950 it is slower than bt_gemv. */
int32_t bt_gemv_lut(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                    const int8_t* x_q, const float* s_a, float* y,
                    int32_t* acc, void* stream);

/* Ternary matrix product: acc[i, r] = sum_k trit(r, k) * x_q[i, k] (exact
 * int32) and y[i, r] = ((float)acc[i, r] * s_w) * s_a[i].
 *  packed  bt_packed_bytes(n, k) bytes from bt_pack_i2s, device, 16-aligned.
 *  s_w     per-tensor weight scale: finite and >= 0.
 *  x_q     int8 [m, k], device, 16-byte aligned;  s_a fp32 [m], device.
 *  y       fp32 [m, n], device, 16-byte aligned.
 *  acc     nullable int32 [m, n], device, 16-byte aligned (parity/debug).
 * Kernel choice by m: m <= 4 uses packed-int8 dot products (v_dot4), larger
 * m uses int8 matrix cores (MFMA). */
int32_t bt_gemm(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                int64_t m, const int8_t* x_q, const float* s_a, float* y,
                int32_t* acc, void* stream);

/* One independent problem of a grouped call (all pointers device). */
typedef struct bt_problem {
  const uint8_t* packed;
  const int8_t* x_q;
  const float* s_a;
  float* y;
  int32_t* acc; /* nullable */
  float s_w;
  int32_t n;
  int32_t k;
  int32_t m; /* every problem of one group has the same m */
} bt_problem;

/* Grouped product: many independent bt_gemm problems in one launch, for a
 * decode step whose projections are each too small to fill the GPU.
 * Use: bytes = bt_grouped_plan_bytes(probs, count); fill a host buffer of that
 * size with bt_grouped_plan (host code: it launches nothing and reads no
 * device memory, and asks the HIP runtime only for the current device's
 * compute-unit count); copy it to device
 * memory the caller owns (256-byte aligned, writable: every launch writes
 * the plan's scratch area); then call bt_gemm_grouped(plan_dev, plan_host, s)
 * as often as wanted.  The plan holds
 * the problem descriptors (pointers, shapes, scales), the work order and a
 * scratch area through which workgroups that share part of the work combine
 * their partial sums: with packed dot products, m * 512 bytes per 64-row
 * block; on the matrix cores, per-range regions and arrival counters for
 * problems whose reduction is split.  The counters and slots are zero in the
 * host image and every complete launch leaves them zero.
 * Hence launches that use one plan must not overlap (use one plan per
 * stream); rebuild the plan when any pointer, shape or scale changes.
 * plan_host must stay a byte-identical copy of the host image written by
 * bt_grouped_plan (only its header is read by bt_gemm_grouped).
 * With packed dot products the plan also records where each wave of a
 * launch on the device that was current when it was built starts streaming
 * (a table sized by that device's compute units; bytes and image must come
 * from calls with the same device current).  A launch on a device with
 * another count gives the same results and finds its starts by a search.
 * Kernel choice: m = 1 streams the weights through packed dot products; so
 * do m = 2 in plans of fewer than 131072 chunks (128 MiB of packed weights)
 * and m = 3, 4 in plans of fewer than 32768 chunks (32 MiB), while larger
 * plans at m = 2..4 and every plan at m > 4 use the int8 matrix cores (the
 * dot products of a large plan are then bound by the vector ALUs, not by the
 * weight stream).
 * bt_grouped_plan_bytes returns the size, or a negative status. */
int64_t bt_grouped_plan_bytes(const bt_problem* probs, int32_t count);
int32_t bt_grouped_plan(const bt_problem* probs, int32_t count, void* plan,
                        int64_t plan_bytes);
int32_t bt_gemm_grouped(void* plan_dev, const void* plan_host,
                        void* stream);

/* bt_grouped_plan with the caller's own per-XCD shares.  A launch whose
 * grid fills the GPU streams each wave's contiguous range of the weights,
 * and the XCDs (each with its own L2 and path to memory; workgroup g runs
 * on XCD g mod nxcd) do not stream equally fast: by default odd XCDs take
 * 0.9 of a share.  Rates measured on the GPU the plan runs on (per-wave
 * timestamps of the timing build, include/bt_timing.h) can be given
 * instead: XCD x's waves then take xcd_permille[x] / 1000 of a share, so
 * that every XCD ends its reads at the same time.  The split changes no
 * output bit.  Shares apply to streaming plans on a full grid of a device
 * with nxcd XCDs and are ignored otherwise (the plan is then that of
 * bt_grouped_plan).  Sizes as bt_grouped_plan_bytes.
 *  xcd_permille  host int32 [nxcd], each in [500, 2000], else BT_E_ARG;
 *                NULL gives BT_E_NULL.
 *  nxcd          1 to 32, else BT_E_ARG. */
int32_t bt_grouped_plan_xcd(const bt_problem* probs, int32_t count,
                            const int32_t* xcd_permille, int32_t nxcd,
                            void* plan, int64_t plan_bytes);

/* bt_gemm_grouped for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launch over the same plan, with the same results bit
 * for bit, except that the scratch memory its kernels use (the partial sums
 * and arrival counters that bt_gemm_grouped keeps in the plan's scratch
 * area) lives in a static array of the library, BT_STATIC_SCRATCH_BYTES per
 * GPU, held from the first call on that GPU until the process ends.  The
 * plan's own scratch area is not touched, so plan_dev may be read-only.
 * Every call zeroes the part of the array its plan uses (one fill kernel on
 * `stream`, before the product) and calls no allocating routine.  All calls
 * on one GPU share its array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results.
 * Returns BT_E_SHAPE when the plan's scratch area (its image size minus the
 * scratch offset in the header) is larger than BT_STATIC_SCRATCH_BYTES;
 * otherwise the checks and results of bt_gemm_grouped. */
#define BT_STATIC_SCRATCH_BYTES (32 << 20)
int32_t bt_gemm_grouped_static(const void* plan_dev, const void* plan_host,
                               void* stream);

/* Grouped decode product that quantizes its own activations (the per-token
 * int8 absmax step and the ternary product in one launch: the 8-bit
 * activation quantization of "BitNet-rs：Rust实现的高效1比特大语言模型推理
 * 引擎", section "技术实现细节", fused into the GEMV).  Each problem gives fp32 activations x [m, k] instead of x_q and
 * s_a; the launch quantizes every token row exactly as bt_quant_act would
 * (same x_q, same s_a, bit for bit) and then computes what bt_gemm would
 * with them.  Neither x_q nor s_a is written out.
 *  x   fp32 [m, k], device, 16-byte aligned.
 * Other fields and rules as in bt_problem, and further 1 <= m <= 4 and
 * m * k <= BT_FUSED_MAX_MK (each wave keeps its problem's quantized rows in
 * LDS); otherwise BT_E_SHAPE.  The plan is launched with bt_gemm_grouped
 * and obeys the same rules (scratch, reuse, no overlapping launches). */
#define BT_FUSED_MAX_MK 16384
typedef struct bt_problem_f32 {
  const uint8_t* packed;
  const float* x;
  float* y;
  int32_t* acc; /* nullable */
  float s_w;
  int32_t n;
  int32_t k;
  int32_t m; /* every problem of one group has the same m */
} bt_problem_f32;
int64_t bt_grouped_plan_f32_bytes(const bt_problem_f32* probs, int32_t count);
int32_t bt_grouped_plan_f32(const bt_problem_f32* probs, int32_t count,
                            void* plan, int64_t plan_bytes);

/* Fewer-bytes format, for comparison: five trits per byte in base 3
 * (1.6 bits per weight, a fifth fewer bytes than bt_pack_i2s when k is a
 * multiple of 80).  The M=1 product is bound by the bytes it reads
 * ("1bit-systems：在AMD Strix Halo上实现纯Rust本地三值权重LLM推理", section
 * "性能实测：92%的内存带宽利用率"), and the CPU kernels of "BitNet 1 位 LLM
 * 独立推理引擎：位串行 GEMM 内核与 LUT 优化工程实践" (body) pack three weights
 * into one index (TL2) to read a sixth fewer bytes; this format takes the
 * same lever further, at the cost of decoding base-3 digits.
 * Layout: rows padded to a multiple of 64 and inputs to a multiple of 80,
 * with trit 0.  Row block b occupies bytes [b * 64 * P * 16,
 * (b + 1) * 64 * P * 16), P = ceil(k / 80); inside it, the 16-byte piece
 * holding inputs [80 p, 80 p + 80) of row r sits at offset
 * (p * 64 + r % 64) * 16; byte 4 u + i of a piece holds inputs
 * 80 p + 20 u + 4 j + i, j = 0..4, as the base-3 number
 * v = sum_j (trit + 1) * 3^(4 - j), stored as ceil(v * 256 / 243).
 * bt_b3_packed_bytes: ceil(n / 64) * 64 * ceil(k / 80) * 16, or BT_E_SHAPE
 * under the rules of bt_packed_bytes.
 * bt_pack_b3: as bt_pack_i2s (same arguments and rules), writing this
 * format; entries outside {-1, 0, 1} are counted in *n_invalid and stored
 * as trit 0.
 * bt_gemv_b3: bt_gemv (same arguments, rules and results, bit for bit) over
 * weights packed by bt_pack_b3. */
int64_t bt_b3_packed_bytes(int64_t n, int64_t k);
int32_t bt_pack_b3(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                   int32_t* n_invalid, void* stream);
int32_t bt_gemv_b3(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                   const int8_t* x_q, const float* s_a, float* y, int32_t* acc,
                   void* stream);

/* Measurement helper, not part of the product path: reads `bytes` of device
 * memory at buf once, with the access pattern of the decode kernel's weight
 * stream (persistent waves, waves_per_cu of them per compute unit, each
 * streaming one contiguous range with non-temporal 128-bit loads, 1 KiB per
 * wave and load, in groups of four loads of which `groups` are in flight),
 * and writes one XOR of the words each wave read to sink[wave].  Timing it
 * gives the streaming-read ceiling of the GPU it runs on, against which the
 * ternary GEMV, a bandwidth-bound kernel ("1bit-systems" page, section
 * "性能实测：92%的内存带宽利用率"), is compared.
 *  buf         device, 16-byte aligned; bytes >= 1024 and bytes % 1024 == 0.
 *  sink        device uint32 [sink_words], 4-byte aligned; sink_words must be
 *              at least (compute units) * waves_per_cu, else BT_E_SHAPE.
 *  waves_per_cu  4 or 8; groups 1 to 4; else BT_E_ARG. */
int32_t bt_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                      int64_t sink_words, int32_t waves_per_cu,
                      int32_t groups, void* stream);

/* Measurement helper, not part of the product path: bt_read_probe with a
 * write stream mixed in.  Besides reading `bytes` at buf once as
 * bt_read_probe does, the waves write out_bytes at out once, in 1 KiB
 * pieces with non-temporal 128-bit stores, each wave its contiguous share,
 * spread evenly through its reads in bursts of `burst` consecutive pieces
 * (the rest at the end of the wave's reads); every 32-bit word of piece i
 * (bytes [1024 i, 1024 i + 1024) of out) receives the value i.  Timing it
 * gives the rate of a memory stream that writes a given fraction of its
 * bytes, as a skinny matrix product writes its outputs between its weight
 * reads.
 *  buf, sink, waves_per_cu, groups  as in bt_read_probe.
 *  out        device, 16-byte aligned (may be NULL when out_bytes is 0);
 *             out_bytes % 1024 == 0 and 0 <= out_bytes <= bytes, else
 *             BT_E_SHAPE.
 *  burst      1 to 64, else BT_E_ARG. */
int32_t bt_mix_probe(const void* buf, int64_t bytes, void* out,
                     int64_t out_bytes, int32_t burst, uint32_t* sink,
                     int64_t sink_words, int32_t waves_per_cu, int32_t groups,
                     void* stream);

/* RMSNorm in front of the activation quantization: RMS normalization is one
 * of the GPU kernels of a ternary model's decode step ("1bit-systems：在AMD
 * Strix Halo上实现纯Rust本地三值权重LLM推理", section "技术架构：Rust在上，HIP
 * 在下").  Per token row x [k] with per-feature gain g [k]:
 * ss = sum x^2 (double accumulation, each square exact), r = (float)(1 /
 * sqrt(ss / k + eps)) (double arithmetic, one rounding), h = (x * r) * g
 * (two fp32 products); then x_q and s_a of h exactly as bt_quant_act gives
 * them.  The sum of squares is taken in one fixed order (lane l of a wave
 * adds float4 l, l + 64, ... in increasing order, lanes combine by an xor
 * butterfly), shared by bt_rmsnorm_quant and the fused plans below, which
 * therefore give the same bits.
 *  x, g   fp32 [m, k] and [k], device, 16-byte aligned.
 *  eps    finite, >= 0, else BT_E_ARG.
 *  x_q, s_a  as in bt_quant_act.
 *  h      nullable fp32 [m, k], device, 16-byte aligned: the normalized
 *         rows, written when given. */
int32_t bt_rmsnorm_quant(const float* x, const float* g, int64_t m, int64_t k,
                         float eps, int8_t* x_q, float* s_a, float* h,
                         void* stream);

/* Grouped decode product with RMSNorm, quantization and product in one
 * launch: as bt_grouped_plan_f32 (same rules, kernel and results), with each
 * problem's fp32 rows first normalized as bt_rmsnorm_quant does (same x_q
 * and s_a, bit for bit).  g must be non-null and 16-byte aligned. */
typedef struct bt_problem_norm {
  const uint8_t* packed;
  const float* x;   /* fp32 [m, k], device, 16-byte aligned */
  const float* g;   /* fp32 [k] gain, device, 16-byte aligned */
  float* y;
  int32_t* acc;     /* nullable */
  float s_w;
  float eps;
  int32_t n;
  int32_t k;
  int32_t m;
} bt_problem_norm;
int64_t bt_grouped_plan_norm_bytes(const bt_problem_norm* probs,
                                   int32_t count);
int32_t bt_grouped_plan_norm(const bt_problem_norm* probs, int32_t count,
                             void* plan, int64_t plan_bytes);

/* Layer-chained decode in one persistent launch: the phases of one token,
 * each a fused plan (bt_grouped_plan_f32 or bt_grouped_plan_norm, one m for
 * all) whose fp32 input may be an output of an earlier phase, run in order
 * in one cooperative launch with a grid-wide barrier between phases.  The
 * results are bit for bit those of launching the plans one after another
 * with bt_gemm_grouped.  (The decode step of a ternary model runs its
 * projections in dependent order: "1bit-systems：在AMD Strix Halo上实现纯
 * Rust本地三值权重LLM推理", section "技术架构：Rust在上，HIP在下", puts the
 * GEMV, RMSNorm and attention kernels of one step behind one native call.)
 * Use: bytes = bt_chain_plan_bytes(count); fill a host buffer with
 * bt_chain_plan from the phases' device plans and host images; copy it to
 * device memory the caller owns (256-byte aligned, writable: every launch
 * zeroes and uses its sync words); launch with bt_gemm_chain.  The plans
 * must stay alive and unchanged; launches of one chain image (or sharing a
 * phase plan) must not overlap.
 * Every wait of the barrier is bounded (0.5 s): if one gives up, the int32
 * at byte BT_CHAIN_STATUS_OFFSET of the device image is nonzero after the
 * launch and the outputs are invalid; it is 0 after a complete launch.
 * Errors: BT_E_ARG for a plan that is not fused or a bad count, BT_E_SHAPE
 * for plans of different m; the launch fails with BT_E_HIP if the GPU cannot
 * hold every workgroup at once. */
#define BT_MAX_CHAIN_PHASES 4096
#define BT_CHAIN_STATUS_OFFSET 4356
typedef struct bt_chain_phase {
  void* plan_dev;         /* device copy of the phase's plan */
  const void* plan_host;  /* its host image */
} bt_chain_phase;
int64_t bt_chain_plan_bytes(int32_t count);
int32_t bt_chain_plan(const bt_chain_phase* phases, int32_t count,
                      void* chain_host, int64_t chain_bytes);
int32_t bt_gemm_chain(void* chain_dev, const void* chain_host, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BT_H */
