// Fewer-bytes ternary GEMV (one token): weights packed five per byte in base
// 3 (1.6 bits per weight instead of 2), kept to measure whether reading a
// fifth fewer bytes pays for the extra decoding on gfx950.
//
// Why: the M=1 product is bound by the bytes it reads ("1bit-systems：在AMD
// Strix Halo上实现纯Rust本地三值权重LLM推理", section "性能实测：92%的内存带宽
// 利用率": only reading fewer bytes makes it faster), and the CPU kernels of
// "BitNet 1 位 LLM 独立推理引擎：位串行 GEMM 内核与 LUT 优化工程实践" (body)
// group three weights into one index (TL2) to read a sixth fewer bytes.  Five
// trits fit one byte because 3^5 = 243 <= 256.
//
// Format (stated in bt.h): a byte stores v = sum_j c_j 3^(4-j) (c = trit + 1)
// as ceil(v * 256 / 243), the base-3 fraction v / 243 scaled to 8 bits.  The
// digits come out most significant first: c_j = (3 x) >> 8, then
// x = (3 x) & 255.  Byte i of a 32-bit word holds inputs 4 j + i (j = 0..4)
// of a 20-input group, so digit j of the word's four bytes lines up with one
// 32-bit word of int8 activations and feeds one v_dot4.
//
// Decoding four bytes at once: the even and the odd bytes go to the two
// 16-bit halves of two registers (3 x < 768, so the halves never carry into
// each other), one multiplication and one mask per register and digit, and
// one byte permutation gathers the four digits.  About 30 vector operations
// per 20 weights, against 9 per 16 for the 2-bit format.
//
// Mapping as in the 2-bit single-problem kernel: a workgroup of WAVES waves
// per 64-row block, lane = row, the waves splitting the row's 16-byte pieces
// (80 inputs each); activations are wave-uniform and come through scalar
// loads; the code offset sum (c - 1) q = sum c q - sum q is applied at the
// end.
#include "bt_internal.h"

namespace bt {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kPieceIn = 80;  // inputs per 16-byte piece

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Byte selection: result byte i is byte sel_i of the 8-byte value whose low
// word is lo and whose high word is hi (selector 12 gives a zero byte).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo,
                                         uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// sum over the word's 20 inputs of digit * activation, for the five
// activation words q[0..4]
__device__ __forceinline__ int dot_word(uint32_t w, const int* q, int acc) {
  uint32_t e = perm(0u, w, 0x0C020C00u);  // bytes 0, 2 -> 16-bit halves
  uint32_t o = perm(0u, w, 0x0C030C01u);  // bytes 1, 3
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    // per half: 3 x < 768, digit j in bits 8-9, the rest of the fraction
    // in bits 0-7
    const uint32_t ey = e * 3u, oy = o * 3u;
    // digit j of bytes 0..3: byte 1 of each half
    const uint32_t c = perm(oy, ey, 0x07030501u);
    acc = sdot4((int)c, q[j], acc);
    e = ey & 0x00FF00FFu;
    o = oy & 0x00FF00FFu;
  }
  return acc;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void b3_kernel(Desc d) {
  __shared__ int red[WAVES][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x;
  const int k = d.k;
  const int P = (k + kPieceIn - 1) / kPieceIn;  // pieces per row
  const int kq = k >> 2;                        // activation words
  const int full = k / kPieceIn;                // pieces with no padding
  const int p0 = P * wave / WAVES, p1 = P * (wave + 1) / WAVES;
  const int pf = min(p1, full);
  const v4u* wp = reinterpret_cast<const v4u*>(d.w) +
                  (size_t)rb * 64 * P + lane;
  const int* q = reinterpret_cast<const int*>(d.xq);
  int acc = 0;
#pragma unroll 2
  for (int p = p0; p < pf; ++p) {
    const v4u wv = __builtin_nontemporal_load(wp + (size_t)p * 64);
    const int* qp = q + 20 * p;  // 20 activation words, all in range
    int qv[20];
#pragma unroll
    for (int i = 0; i < 20; ++i) qv[i] = qp[i];
    acc = dot_word(wv.x, qv, acc);
    acc = dot_word(wv.y, qv + 5, acc);
    acc = dot_word(wv.z, qv + 10, acc);
    acc = dot_word(wv.w, qv + 15, acc);
  }
  if (p1 > full && p0 <= full) {
    // the padded last piece (k % 80 != 0): activation words past the row
    // read as zero; their weights are trit 0 (digit 1) and add nothing
    const int p = full;
    const v4u wv = __builtin_nontemporal_load(wp + (size_t)p * 64);
    int qv[20];
#pragma unroll
    for (int i = 0; i < 20; ++i) {
      const int idx = 20 * p + i;
      const int v = q[min(idx, kq - 1)];
      qv[i] = idx < kq ? v : 0;
    }
    acc = dot_word(wv.x, qv, acc);
    acc = dot_word(wv.y, qv + 5, acc);
    acc = dot_word(wv.z, qv + 10, acc);
    acc = dot_word(wv.w, qv + 15, acc);
  }
  // activation sum over this wave's inputs (the code offset)
  const int w0 = 20 * p0, w1 = min(20 * p1, kq);
  int s = 0;
  for (int i = w0 + lane; i < w1; i += 64) s = sdot4(q[i], 0x01010101, s);
  red[wave][lane] = acc - wave_sum(s);
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

// One thread per (row, piece): reads the piece's 80 trits of its row (trit 0
// past the row's end and for padding rows) and writes 16 bytes.  Thread
// index L = (row block * P + piece) * 64 + row % 64 is the piece's position
// in the output, so the stores coalesce.
__global__ __launch_bounds__(256) void pack_b3_kernel(
    const int8_t* __restrict__ t, int64_t n, int64_t k, int64_t total,
    uint8_t* __restrict__ packed, int32_t* n_invalid) {
  const int64_t L = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t P = (k + kPieceIn - 1) / kPieceIn;
  int bad = 0;
  if (L < total) {
    const int64_t r = (L / (64 * P)) * 64 + (L & 63);
    const int64_t p = (L >> 6) % P;
    const int8_t* row = t + r * k;
    uint32_t words[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int v = 0;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const int64_t c = p * kPieceIn + 20 * u + 4 * j + i;
          int code = 1;
          if (r < n && c < k) {
            const int tv = row[c];
            if (tv >= -1 && tv <= 1)
              code = tv + 1;
            else
              ++bad;
          }
          v = 3 * v + code;
        }
        word |= (uint32_t)((v * 256 + 242) / 243) << (8 * i);
      }
      words[u] = word;
    }
    reinterpret_cast<v4u*>(packed)[L] = v4u{words[0], words[1], words[2],
                                            words[3]};
  }
  if (n_invalid != nullptr) {
    bad = wave_sum(bad);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(n_invalid, bad);
  }
}

template <int WAVES>
hipError_t launch_b3_waves(const Desc& d, hipStream_t s) {
  b3_kernel<WAVES><<<dim3((unsigned)d.nblk), dim3(64 * WAVES), 0, s>>>(d);
  return hipGetLastError();
}

}  // namespace

int64_t b3_packed_bytes(int64_t n, int64_t k) {
  return (n + 63) / 64 * 64 * ((k + kPieceIn - 1) / kPieceIn) * 16;
}

hipError_t launch_pack_b3(const int8_t* t, int64_t n, int64_t k,
                          uint8_t* packed, int32_t* n_invalid, hipStream_t s) {
  const int64_t total = b3_packed_bytes(n, k) / 16;
  pack_b3_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
      t, n, k, total, packed, n_invalid);
  return hipGetLastError();
}

hipError_t launch_b3(const Desc& d, hipStream_t s) {
  const int pieces = (d.k + kPieceIn - 1) / kPieceIn;
  // the 2-bit kernel's rule, counted in pieces of 80 inputs
  switch (row_block_waves(d.nblk, pieces)) {
    case 16: return launch_b3_waves<16>(d, s);
    case 8: return launch_b3_waves<8>(d, s);
    default: return launch_b3_waves<4>(d, s);
  }
}

}  // namespace bt
