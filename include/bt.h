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
 * size with bt_grouped_plan (pure host code, no HIP call); copy it to device
 * memory the caller owns (256-byte aligned); then call
 * bt_gemm_grouped(plan_dev, plan_host, s) as often as wanted.  The plan holds
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
int32_t bt_gemm_grouped(const void* plan_dev, const void* plan_host,
                        void* stream);

/* Grouped decode product that quantizes its own activations (the per-token
 * int8 absmax step and the ternary product in one launch: the activation
 * quantization of "Microsoft BitNet" section "技术实现细节" fused into the
 * GEMV).  Each problem gives fp32 activations x [m, k] instead of x_q and
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

#ifdef __cplusplus
}
#endif
#endif /* BT_H */
