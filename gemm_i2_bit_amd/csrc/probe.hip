// Streaming-read probe: the HBM read rate that a pure sequential read of a
// device buffer reaches on this GPU, measured with the same access pattern as
// the decode kernel's weight stream (persistent waves, each streaming one
// contiguous range in 1 KiB steps with non-temporal 128-bit buffer loads, in
// groups of four loads, 1 to 4 groups in flight).  The ternary GEMV is bound by this rate
// ("1bit-systems" page, section "性能实测：92%的内存带宽利用率": the GEMV
// saturates memory bandwidth), so the benchmark reports its products as a
// fraction of the nameplate peak and of this measured ceiling.  Nothing of
// the product path uses this kernel.
#include "bt_internal.h"

namespace bt {
#ifdef BT_WAVE_TIMESTAMPS
// Timing build only: per wave of the last probe launch, the real-time
// counter at entry (slot 0), when its first load group has arrived (1) and
// at the end of its loop (2), and its hardware position.
__device__ unsigned long long g_probe_ts[kTimedWaves * 4];
__device__ unsigned int g_probe_hw[kTimedWaves * 2];
__device__ __forceinline__ void probe_stamp(int64_t wv, int slot) {
  const unsigned long long t = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0 && wv < kTimedWaves) {
    g_probe_ts[wv * 4 + slot] = t;
    if (slot == 0) {
      g_probe_hw[wv * 2] = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
      g_probe_hw[wv * 2 + 1] =
          __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));
    }
  }
}
#endif
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit words
constexpr int D = 4;                     // 1 KiB steps per load group

__device__ __forceinline__ void load_group(v4u (&buf)[D], const uint8_t* base,
                                           int64_t chunk, int cnt) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + chunk * 1024), 0, cnt * 1024, kRsrcFlags);
  const int lane16 = (threadIdx.x & 63) * 16;
#pragma unroll
  for (int j = 0; j < D; ++j)
    buf[j] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(r, lane16 + j * 1024, 0, 2));
}

// Steps of a group starting at step `at` of a range ending at `hi` (0..D).
__device__ __forceinline__ int group_cnt(int64_t at, int64_t hi) {
  const int64_t left = hi - at;
  return left <= 0 ? 0 : (left >= D ? D : (int)left);
}

__device__ __forceinline__ uint32_t fold(const v4u (&buf)[D]) {
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < D; ++j) x ^= buf[j].x ^ buf[j].y ^ buf[j].z ^ buf[j].w;
  return x;
}

// Wave w of W reads 1 KiB steps [w T / W, (w + 1) T / W), with G groups of
// D loads in flight, and writes the XOR of every word it read to sink[w]
// (so that no load is dead).
template <int WPW, int G>
__global__ __launch_bounds__(64 * WPW) void read_probe_kernel(
    const uint8_t* __restrict__ buf, int64_t total, uint32_t* sink) {
  const int64_t W = (int64_t)gridDim.x * WPW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wv = (int64_t)blockIdx.x * WPW + wave;
  const int64_t lo = wv * total / W, hi = (wv + 1) * total / W;
#ifdef BT_WAVE_TIMESTAMPS
  probe_stamp(wv, 0);
#endif
  uint32_t x = 0;
  v4u ring[G][D];
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(ring[g], buf, lo + g * D,
                                         group_cnt(lo + g * D, hi));
#ifdef BT_WAVE_TIMESTAMPS
  {  // the first group's loads have arrived (the wait the first fold makes)
    constexpr int n = (G - 1) * D;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) |
                               ((n >> 4) << 14));
    probe_stamp(wv, 1);
  }
#endif
  for (int64_t pos = lo; pos < hi; pos += G * D) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // group g of this round holds steps pos + g D ..; once folded, its
      // buffer takes the group G rounds ahead
      x ^= fold(ring[g]);
      const int64_t next = pos + (g + G) * D;
      load_group(ring[g], buf, next, group_cnt(next, hi));
    }
  }
#ifdef BT_WAVE_TIMESTAMPS
  probe_stamp(wv, 2);
#endif
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) sink[wv] = x;
}

// The read probe with a write stream mixed in: wave w also writes its share
// [w P / W, (w + 1) P / W) of the P 1 KiB pieces of `out`, spread evenly
// through its reads in bursts of `burst` pieces (after a load group is
// issued, once that many pieces are due; the rest after its last reads),
// with non-temporal 128-bit stores, each piece filled with its own index.  Timing it gives the rate of a stream that
// writes a given fraction of its bytes, as a skinny matrix product writes
// its outputs between its weight reads (a tile's outputs in one burst).
template <int WPW, int G>
__global__ __launch_bounds__(64 * WPW) void mix_probe_kernel(
    const uint8_t* __restrict__ buf, int64_t total, uint32_t* __restrict__ out,
    int64_t pieces, int burst, uint32_t* sink) {
  const int64_t W = (int64_t)gridDim.x * WPW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wv = (int64_t)blockIdx.x * WPW + wave;
  const int64_t lo = wv * total / W, hi = (wv + 1) * total / W;
  const int64_t wlo = wv * pieces / W, whi = (wv + 1) * pieces / W;
  const int lane = threadIdx.x & 63;
  int64_t wnext = wlo;
  typedef __attribute__((address_space(1))) v4u* gv4u_ptr;
  typedef __attribute__((address_space(1))) uint32_t* gu32_ptr;
  uint32_t x = 0;
  v4u ring[G][D];
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(ring[g], buf, lo + g * D,
                                         group_cnt(lo + g * D, hi));
  for (int64_t pos = lo; pos < hi; pos += G * D) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      x ^= fold(ring[g]);
      const int64_t next = pos + (g + G) * D;
      load_group(ring[g], buf, next, group_cnt(next, hi));
      // pieces due once steps [lo, pos + (g + 1) D) are read
      const int64_t done = min(pos + (g + 1) * D, hi) - lo;
      const int64_t due = wlo + (whi - wlo) * done / (hi - lo);
      if (due - wnext < burst) continue;
      for (; wnext < due; ++wnext) {
        const uint32_t v = (uint32_t)wnext;
        __builtin_nontemporal_store(
            v4u{v, v, v, v},
            reinterpret_cast<gv4u_ptr>((gu32_ptr)(out + wnext * 256 + lane * 4)));
      }
    }
  }
  for (; wnext < whi; ++wnext) {
    const uint32_t v = (uint32_t)wnext;
    __builtin_nontemporal_store(
        v4u{v, v, v, v},
        reinterpret_cast<gv4u_ptr>((gu32_ptr)(out + wnext * 256 + lane * 4)));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if (lane == 0) sink[wv] = x;
}

template <int WPW>
void launch_mix_wpw(const uint8_t* b, int64_t steps, uint32_t* out,
                    int64_t pieces, int burst, uint32_t* sink, int waves,
                    int groups, hipStream_t s) {
  const dim3 grid((unsigned)(waves / WPW)), block(64 * WPW);
  switch (groups) {
    case 1: mix_probe_kernel<WPW, 1><<<grid, block, 0, s>>>(b, steps, out, pieces, burst, sink); break;
    case 2: mix_probe_kernel<WPW, 2><<<grid, block, 0, s>>>(b, steps, out, pieces, burst, sink); break;
    case 3: mix_probe_kernel<WPW, 3><<<grid, block, 0, s>>>(b, steps, out, pieces, burst, sink); break;
    default: mix_probe_kernel<WPW, 4><<<grid, block, 0, s>>>(b, steps, out, pieces, burst, sink); break;
  }
}

template <int WPW>
void launch_wpw(const uint8_t* b, int64_t steps, uint32_t* sink, int waves,
                int groups, hipStream_t s) {
  const dim3 grid((unsigned)(waves / WPW)), block(64 * WPW);
  switch (groups) {
    case 1: read_probe_kernel<WPW, 1><<<grid, block, 0, s>>>(b, steps, sink); break;
    case 2: read_probe_kernel<WPW, 2><<<grid, block, 0, s>>>(b, steps, sink); break;
    case 3: read_probe_kernel<WPW, 3><<<grid, block, 0, s>>>(b, steps, sink); break;
    default: read_probe_kernel<WPW, 4><<<grid, block, 0, s>>>(b, steps, sink); break;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                             int waves, int wpw, int groups, hipStream_t s) {
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (wpw == 8)
    launch_wpw<8>(b, bytes / 1024, sink, waves, groups, s);
  else
    launch_wpw<4>(b, bytes / 1024, sink, waves, groups, s);
  return hipGetLastError();
}

hipError_t launch_mix_probe(const void* buf, int64_t bytes, void* out,
                            int64_t out_bytes, int burst, uint32_t* sink,
                            int waves, int wpw, int groups, hipStream_t s) {
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  uint32_t* o = static_cast<uint32_t*>(out);
  if (wpw == 8)
    launch_mix_wpw<8>(b, bytes / 1024, o, out_bytes / 1024, burst, sink,
                      waves, groups, s);
  else
    launch_mix_wpw<4>(b, bytes / 1024, o, out_bytes / 1024, burst, sink,
                      waves, groups, s);
  return hipGetLastError();
}

}  // namespace bt

#ifdef BT_WAVE_TIMESTAMPS
extern "C" int32_t bt_probe_timestamps(uint64_t* ts, uint32_t* hw) {
  if (!ts || !hw) return BT_E_NULL;
  if (hipMemcpyFromSymbol(ts, HIP_SYMBOL(bt::g_probe_ts),
                          sizeof(bt::g_probe_ts)) != hipSuccess ||
      hipMemcpyFromSymbol(hw, HIP_SYMBOL(bt::g_probe_hw),
                          sizeof(bt::g_probe_hw)) != hipSuccess)
    return BT_E_HIP;
  return BT_OK;
}
#endif
