/*
 * Oracle for the W1.58A8 ternary matrix product: a plain, slow, obviously
 * correct CPU implementation.  TEST INFRASTRUCTURE ONLY: it is used by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *  - "1bit-systems：在AMD Strix Halo上实现纯Rust本地三值权重LLM推理",
 *    section "三值量化：1.58-bit的魔法": weights take one of -1, 0, +1.
 *  - bitnet.cpp CPU tutorial (m.qwbw.cn/news/64613), §1.1: ternary weights,
 *    stored 2 bits each in practice; a multiply by -1/0/+1 is negate/skip/copy,
 *    so the product is a sign test plus accumulation.
 *  - same tutorial, §3.2: conversion projects every weight onto the ternary
 *    set by absmean quantization.
 *  - "BitNet-rs：Rust实现的高效1比特大语言模型推理引擎", section
 *    "技术实现细节": activations are quantized to 8 bits.
 *  - "BitNet 1 位 LLM 独立推理引擎：位串行 GEMM 内核与 LUT 优化工程实践",
 *    body paragraph on conversion: the generic 2-bit format is called I2_S.
 * The pages fix no bit layout, rounding rule or scale formula; the readings
 * used here (code = trit + 1, the word-interleaved 2-bit layout, round half to
 * even, clamp to +-127, amax floor 1e-5, x * (127 / amax)) are listed with the
 * reasons in the design notes of this repository.
 */
#ifndef BT_ORACLE_H
#define BT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* O1: absmean ternarization of an fp32 [n, k] tensor.
 * gamma = (float)(sum |w| / (n k)) with the sum in double; t = clamp(rne(w /
 * gamma), -1, 1) with an fp32 divide; *s_w = gamma.  gamma == 0 gives t = 0.
 * Returns 0. */
int oracle_ternarize_absmean(const float* w, int64_t n, int64_t k, int8_t* t,
                             float* s_w);

/* O2: pack trits [n, k] (k % 64 == 0) into the 64-row-tiled 2-bit layout.
 * Code c = t + 1 in {0, 1, 2}.  Rows are padded to np = ceil(n / 64) * 64;
 * padding rows hold code 1 (trit 0).  Row block b = r / 64 occupies bytes
 * [b * 16 k, (b + 1) * 16 k); inside it, 16-byte chunk c = k / 64 of row
 * r % 64 sits at offset c * 1024 + (r % 64) * 16; inside the chunk, weight k
 * sits in byte 4 ((k % 64) / 16) + (k % 4) at bit 2 ((k % 16) / 4).
 * Total size np * k / 4 bytes.  Returns the number of entries outside
 * {-1, 0, 1}; such entries are stored as code 3 (no trit maps to it). */
int64_t oracle_pack_i2s(const int8_t* t, int64_t n, int64_t k, uint8_t* packed);

/* O2 inverse: unpack the first n rows to trits.  Code 3 is invalid: it is
 * written as the value 2 (not a trit) and counted; returns the count. */
int64_t oracle_unpack_i2s(const uint8_t* packed, int64_t n, int64_t k,
                          int8_t* t);

/* Fewer-bytes packing (base 3, five trits per byte), the comparison format
 * of the "fewer bytes" lever: "1bit-systems：在AMD Strix Halo上实现纯Rust本地
 * 三值权重LLM推理", section "性能实测：92%的内存带宽利用率" (the GEMV is bound
 * by the bytes it reads), and "BitNet 1 位 LLM 独立推理引擎：位串行 GEMM 内核
 * 与 LUT 优化工程实践" (body: TL2 groups three weights into one index and
 * needs a sixth less bandwidth than 2 bits per weight).  Five trits per byte
 * is 1.6 bits per weight: 3^5 = 243 <= 256.
 * Layout: rows padded to np = ceil(n / 64) * 64 (trit 0); inputs padded to
 * kp = ceil(k / 80) * 80 (trit 0).  Row block b = r / 64 occupies bytes
 * [b * 64 * kp / 5, (b + 1) * 64 * kp / 5); inside it the 16-byte piece
 * holding inputs [80 p, 80 p + 80) of row r sits at offset
 * (p * 64 + r % 64) * 16.  Inside a piece, byte 4 u + i (u < 4, i < 4) holds
 * the five inputs 80 p + 20 u + 4 j + i, j = 0..4, as the base-3 number
 * v = sum_j c_j * 3^(4 - j) (c = trit + 1, j = 0 most significant), stored
 * as the byte ceil(v * 256 / 243).  Decoding a byte x: for j = 0..4,
 * c_j = (3 x) >> 8 and x = (3 x) & 255.  Returns the number of entries
 * outside {-1, 0, 1}; they are encoded as trit 0. */
int64_t oracle_b3_packed_bytes(int64_t n, int64_t k);
int64_t oracle_pack_b3(const int8_t* t, int64_t n, int64_t k, uint8_t* packed);
/* Inverse of oracle_pack_b3 for the first n rows and k inputs.  A byte whose
 * decoded digits do not re-encode to it (not produced by the packer) is
 * counted; returns the count. */
int64_t oracle_unpack_b3(const uint8_t* packed, int64_t n, int64_t k,
                         int8_t* t);

/* O3: per-row (per token) absmax quantization of fp32 x [m, k] to int8.
 * amax = max |x|, a = max(amax, 1e-5f), inv = 127.0f / a (fp32),
 * q = clamp(rne(x * inv), -127, 127) (fp32 product), s_a = a / 127.0f. */
int oracle_quant_act(const float* x, int64_t m, int64_t k, int8_t* q,
                     float* s_a);

/* RMSNorm in front of the activation quantization (the fused prologue; RMS
 * normalization is one of the hand-written GPU kernels of "1bit-systems：在
 * AMD Strix Halo上实现纯Rust本地三值权重LLM推理", section "技术架构：Rust在
 * 上，HIP在下").  Per row of x [m, k] with per-feature gain g [k]:
 * ss = sum x^2 accumulated in double (each square exact), taken in index
 * order; r64 = 1 / sqrt(ss / k + eps) in double; r = (float)r64;
 * h = (x * r) * g with two fp32 products.  r64[i] receives r64 (nullable).
 * Returns 0. */
int oracle_rmsnorm(const float* x, const float* g, int64_t m, int64_t k,
                   float eps, float* h, double* r64);

/* O4 + O5: acc[i, r] = sum_k trit(r, k) * q[i, k], exact (int64 sum, checked
 * to fit int32); y[i, r] = acc * s_w * s_a[i] evaluated in double.
 * packed holds n rows in the O2 layout, q is [m, k].  Only output rows
 * r0 <= r < r1 are computed; acc and y are [m, r1 - r0] (either may be NULL).
 * The rows are split over `nthreads` threads in contiguous slices; each
 * output is computed by the same plain loop.
 * Returns 0, -1 if an accumulator left int32, -2 on an invalid code. */
int oracle_gemm(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                int64_t m, const int8_t* q, const float* s_a, int64_t r0,
                int64_t r1, int32_t* acc, double* y, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
