/*
 * Oracle for the W1.58A8 ternary matrix product (plain C, scalar loops).
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg.  It shares no code with the HIP library.
 * Every function states the passage it follows; the header lists the readings
 * taken where the pages are silent.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 *        -pthread (no FMA contraction, IEEE single precision for float).
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

/* --- O1: absmean ternarization ------------------------------------------
 * bitnet.cpp CPU tutorial (m.qwbw.cn), §3.2: the converter projects all
 * weights onto {-1, 0, +1} by absmean quantization: divide by the mean
 * absolute value and round to the nearest of the three values. */
int oracle_ternarize_absmean(const float* w, int64_t n, int64_t k, int8_t* t,
                             float* s_w) {
  const int64_t count = n * k;
  double sum = 0.0;
  for (int64_t i = 0; i < count; ++i) sum += fabs((double)w[i]);
  const float gamma = (float)(sum / (double)count);
  *s_w = gamma;
  for (int64_t i = 0; i < count; ++i) {
    if (gamma == 0.0f) {
      t[i] = 0;
      continue;
    }
    const float scaled = w[i] / gamma;       /* fp32 divide */
    float r = nearbyintf(scaled);            /* round half to even */
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    t[i] = (int8_t)r;
  }
  return 0;
}

/* --- O2: 2-bit packing ---------------------------------------------------
 * bitnet.cpp CPU tutorial, §1.1: each ternary weight is stored in 2 bits.
 * "BitNet 1 位 LLM 独立推理引擎" (conversion paragraph): this generic 2-bit
 * format is I2_S.  The byte layout is this library's reading (header). */
static int64_t offset_of(int64_t r, int64_t c, int64_t k) {
  return (r / 64) * 16 * k + (c / 64) * 1024 + (r % 64) * 16 +
         4 * ((c % 64) / 16) + (c % 4);
}
static int shift_of(int64_t c) { return (int)(2 * ((c % 16) / 4)); }

int64_t oracle_pack_i2s(const int8_t* t, int64_t n, int64_t k,
                        uint8_t* packed) {
  const int64_t rows_padded = (n + 63) / 64 * 64;
  int64_t invalid = 0;
  for (int64_t i = 0; i < rows_padded * k / 4; ++i) packed[i] = 0;
  for (int64_t r = 0; r < rows_padded; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      unsigned code = 1;                       /* padding rows: trit 0 */
      if (r < n) {
        const int8_t v = t[r * k + c];
        if (v == -1) code = 0;
        else if (v == 0) code = 1;
        else if (v == 1) code = 2;
        else { code = 3; ++invalid; }
      }
      packed[offset_of(r, c, k)] |= (uint8_t)(code << shift_of(c));
    }
  }
  return invalid;
}

int64_t oracle_unpack_i2s(const uint8_t* packed, int64_t n, int64_t k,
                          int8_t* t) {
  int64_t invalid = 0;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      const unsigned code = (packed[offset_of(r, c, k)] >> shift_of(c)) & 3u;
      if (code == 3) { ++invalid; t[r * k + c] = 2; }
      else t[r * k + c] = (int8_t)((int)code - 1);
    }
  }
  return invalid;
}

/* --- Fewer-bytes packing: five trits per byte (base 3) ------------------
 * "1bit-systems" page, section "性能实测：92%的内存带宽利用率": the GEMV only
 * gets faster by reading fewer bytes.  "BitNet 1 位 LLM 独立推理引擎" (body):
 * TL2 packs three weights into one 5-bit index, a sixth fewer bytes than
 * 2 bits per weight.  Here five trits share one byte as a base-3 number (the
 * layout is stated in the header). */
int64_t oracle_b3_packed_bytes(int64_t n, int64_t k) {
  return (n + 63) / 64 * 64 * ((k + 79) / 80) * 16;
}

static int64_t b3_offset(int64_t r, int64_t c, int64_t k, int* digit) {
  const int64_t pieces = (k + 79) / 80;
  const int64_t p = c / 80, in = c % 80;
  const int64_t u = in / 20, j = (in % 20) / 4, i = in % 4;
  *digit = (int)j;
  return (r / 64) * 64 * pieces * 16 + (p * 64 + r % 64) * 16 + 4 * u + i;
}

int64_t oracle_pack_b3(const int8_t* t, int64_t n, int64_t k,
                       uint8_t* packed) {
  const int64_t rows_padded = (n + 63) / 64 * 64;
  const int64_t kp = (k + 79) / 80 * 80;
  const int64_t bytes = oracle_b3_packed_bytes(n, k);
  int64_t invalid = 0;
  /* first the base-3 value of every byte, then its scaled encoding */
  int32_t* v = (int32_t*)calloc((size_t)bytes, sizeof(int32_t));
  static const int pow3[5] = {81, 27, 9, 3, 1};
  for (int64_t r = 0; r < rows_padded; ++r) {
    for (int64_t c = 0; c < kp; ++c) {
      int code = 1;                       /* padding: trit 0 */
      if (r < n && c < k) {
        const int8_t x = t[r * k + c];
        if (x >= -1 && x <= 1) code = x + 1;
        else ++invalid;
      }
      int digit;
      const int64_t o = b3_offset(r, c, k, &digit);
      v[o] += code * pow3[digit];
    }
  }
  for (int64_t o = 0; o < bytes; ++o)
    packed[o] = (uint8_t)((v[o] * 256 + 242) / 243);  /* ceil(v * 256 / 243) */
  free(v);
  return invalid;
}

int64_t oracle_unpack_b3(const uint8_t* packed, int64_t n, int64_t k,
                         int8_t* t) {
  int64_t bad = 0;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      int digit;
      const int64_t o = b3_offset(r, c, k, &digit);
      unsigned x = packed[o], code = 0;
      for (int j = 0; j <= digit; ++j) {
        code = (3u * x) >> 8;
        x = (3u * x) & 255u;
      }
      t[r * k + c] = (int8_t)((int)code - 1);
    }
  }
  /* bytes the packer cannot have written: decode, re-encode, compare */
  const int64_t bytes = oracle_b3_packed_bytes(n, k);
  for (int64_t o = 0; o < bytes; ++o) {
    unsigned x = packed[o], v = 0;
    for (int j = 0; j < 5; ++j) {
      v = 3u * v + ((3u * x) >> 8);
      x = (3u * x) & 255u;
    }
    if ((v * 256u + 242u) / 243u != packed[o] || v > 242u) ++bad;
  }
  return bad;
}

/* --- O3: per-token absmax int8 quantization ------------------------------
 * "BitNet-rs" page, section "技术实现细节": activations are quantized to 8
 * bits.  Per token, the largest magnitude maps to 127 and every element is
 * scaled by the same factor and rounded (readings in the header). */
int oracle_quant_act(const float* x, int64_t m, int64_t k, int8_t* q,
                     float* s_a) {
  for (int64_t i = 0; i < m; ++i) {
    const float* row = x + i * k;
    float amax = 0.0f;
    for (int64_t c = 0; c < k; ++c) {
      const float mag = fabsf(row[c]);
      if (mag > amax) amax = mag;
    }
    const float a = amax > 1e-5f ? amax : 1e-5f;
    const float inv = 127.0f / a;            /* fp32, correctly rounded */
    for (int64_t c = 0; c < k; ++c) {
      const float p = row[c] * inv;          /* fp32 product */
      float r = nearbyintf(p);               /* round half to even */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[i * k + c] = (int8_t)r;
    }
    s_a[i] = a / 127.0f;
  }
  return 0;
}

/* --- RMSNorm before the quantization -------------------------------------
 * "1bit-systems" page, section "技术架构：Rust在上，HIP在下": RMS
 * normalization is one of the GPU kernels of the decode step.  Each row is
 * divided by the root of its mean square (plus eps) and scaled by the
 * per-feature gain; the precision of each step is the reading stated in the
 * header. */
int oracle_rmsnorm(const float* x, const float* g, int64_t m, int64_t k,
                   float eps, float* h, double* r64) {
  for (int64_t i = 0; i < m; ++i) {
    const float* row = x + i * k;
    double ss = 0.0;
    for (int64_t c = 0; c < k; ++c) ss += (double)row[c] * (double)row[c];
    const double rr = 1.0 / sqrt(ss / (double)k + (double)eps);
    const float r = (float)rr;
    if (r64) r64[i] = rr;
    for (int64_t c = 0; c < k; ++c) {
      const float xr = row[c] * r;  /* fp32 product */
      h[i * k + c] = xr * g[c];     /* fp32 product */
    }
  }
  return 0;
}

/* --- O4 + O5: exact integer contraction, then the rescale ----------------
 * bitnet.cpp CPU tutorial, §1.1: with weights in {-1, 0, +1} every product
 * is the activation, its negation or nothing, so the matrix product is a
 * sign test plus accumulation.  The output is that integer times the weight
 * scale times the token's activation scale. */
typedef struct {
  const uint8_t* packed;
  float s_w;
  int64_t k, m, width, base;
  const int8_t* q;
  const float* s_a;
  int32_t* acc;
  double* y;
  int64_t r0, r1;
  int status;
} gemm_job;

static void* gemm_rows(void* arg) {
  gemm_job* j = (gemm_job*)arg;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    for (int64_t i = 0; i < j->m; ++i) {
      int64_t sum = 0;
      for (int64_t c = 0; c < j->k; ++c) {
        const unsigned code =
            (j->packed[offset_of(r, c, j->k)] >> shift_of(c)) & 3u;
        if (code == 3) { j->status = -2; return NULL; }
        const int64_t trit = (int64_t)code - 1;
        sum += trit * (int64_t)j->q[i * j->k + c];
      }
      if (sum > INT32_MAX || sum < INT32_MIN) { j->status = -1; return NULL; }
      const int64_t out = i * j->width + (r - j->base);
      if (j->acc) j->acc[out] = (int32_t)sum;
      if (j->y) j->y[out] = (double)sum * (double)j->s_w * (double)j->s_a[i];
    }
  }
  return NULL;
}

int oracle_gemm(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                int64_t m, const int8_t* q, const float* s_a, int64_t r0,
                int64_t r1, int32_t* acc, double* y, int nthreads) {
  if (r0 < 0 || r1 > n || r0 > r1) return -3;
  const int64_t rows = r1 - r0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  gemm_job* jobs = (gemm_job*)calloc((size_t)nthreads, sizeof(gemm_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; ++t) {
    gemm_job* j = &jobs[t];
    j->packed = packed; j->s_w = s_w; j->k = k; j->m = m;
    j->width = rows; j->base = r0;
    j->q = q; j->s_a = s_a; j->acc = acc; j->y = y;
    j->r0 = r0 + rows * t / nthreads;
    j->r1 = r0 + rows * (t + 1) / nthreads;
    j->status = 0;
    if (t > 0) pthread_create(&tids[t], NULL, gemm_rows, j);
  }
  gemm_rows(&jobs[0]);
  int status = jobs[0].status;
  for (int t = 1; t < nthreads; ++t) {
    pthread_join(tids[t], NULL);
    if (jobs[t].status != 0) status = jobs[t].status;
  }
  free(jobs);
  free(tids);
  return status;
}
