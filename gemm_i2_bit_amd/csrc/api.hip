// C ABI entry points: host-side argument checks, grouped work plans and
// kernel dispatch.  Declarations and the contract are in bt.h.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <vector>

#include "bt_internal.h"

using bt::Desc;
using bt::PlanHeader;
using bt::Unit;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];   // compute units, 0 = unknown
std::atomic<int> g_xccs[kMaxDevices];  // XCDs, 0 = unknown

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool k_ok(int64_t k) { return k >= 64 && k % 64 == 0 && k <= BT_MAX_K; }
bool n_ok(int64_t n) { return n >= 1 && n <= BT_MAX_N; }
bool m_ok(int64_t m) { return m >= 1 && m <= BT_MAX_M; }

int32_t check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BT_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BT_E_ARCH;
  int state = g_arch[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BT_E_HIP;
    const char* name = prop.gcnArchName;
    const bool ok = strncmp(name, "gfx950", 6) == 0 &&
                    (name[6] == '\0' || name[6] == ':');
    state = ok ? 1 : 2;
    g_arch[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? BT_OK : BT_E_ARCH;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? BT_OK : BT_E_HIP; }

// Compute units of the current device (cached); 0 on error.
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 0;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess)
      return 0;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// XCDs (accelerator complex dies) of the current device (cached); 0 on
// error.
int xcc_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 0;
  int x = g_xccs[dev].load(std::memory_order_relaxed);
  if (x == 0) {
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) !=
        hipSuccess)
      return 0;
    g_xccs[dev].store(x, std::memory_order_relaxed);
  }
  return x;
}

// Checks shared by bt_gemm and the grouped plan.
int32_t check_problem(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                      int64_t m, const int8_t* x_q, const float* s_a,
                      const float* y, const int32_t* acc) {
  if (!packed || !x_q || !s_a || !y) return BT_E_NULL;
  if (!n_ok(n) || !k_ok(k) || !m_ok(m)) return BT_E_SHAPE;
  // chunk indices inside one problem and grids stay 32-bit
  if ((n + 63) / 64 * (k / 64) >= INT32_MAX ||
      bt::kind_units(bt::plan_kind(m), n, m) >= INT32_MAX / 4)
    return BT_E_SHAPE;
  if (!aligned(packed, 16) || !aligned(x_q, 16) || !aligned(y, 16) ||
      !aligned(s_a, 4) || (acc && !aligned(acc, 16)))
    return BT_E_ALIGN;
  if (!std::isfinite(s_w) || s_w < 0.0f) return BT_E_ARG;
  return BT_OK;
}

Desc make_desc(const uint8_t* packed, float s_w, int64_t n, int64_t k,
               int64_t m, const int8_t* x_q, const float* s_a, float* y,
               int32_t* acc) {
  Desc d;
  memset(&d, 0, sizeof(d));
  d.w = packed;
  d.xq = x_q;
  d.sa = s_a;
  d.y = y;
  d.acc = acc;
  d.sw = s_w;
  d.n = (int32_t)n;
  d.k = (int32_t)k;
  d.m = (int32_t)m;
  d.nblk = (int32_t)((n + 63) / 64);
  d.ntt = (int32_t)((m + bt::token_tile(m) - 1) / bt::token_tile(m));
  d.kc = (int32_t)(k / 64);
  d.nsplit = 1;
  d.split_len = d.kc;
  d.slot0 = -1;
  d.region0 = -1;
  return d;
}

// Reduction split of each problem of a matrix-core plan.  Prefill tiles are
// bound by the matrix cores and one tile runs per workgroup, so a problem
// with a long reduction would finish last: its tiles are cut into ranges of
// about the shortest problem's chunk count, but not below kMinSplit chunks
// (a tiny problem in the plan must not cut the others into ranges whose
// set-up and combining outweigh their work), and always an even number of
// chunks, so that only the last range of a row can end on an odd chunk.
constexpr int32_t kMinSplit = 32;
struct Split {
  int32_t nsplit, len;
};
std::vector<Split> plan_splits(const bt_problem* probs, int32_t count,
                               int kind) {
  std::vector<Split> out(count);
  int32_t kc_min = INT32_MAX;
  for (int32_t i = 0; i < count; ++i)
    kc_min = std::min(kc_min, (int32_t)(probs[i].k / 64));
  kc_min = std::max(kc_min, kMinSplit);
  for (int32_t i = 0; i < count; ++i) {
    const int32_t kc = probs[i].k / 64;
    int32_t ns = 1;
    if (kind == bt::kKindPrefill) ns = std::max(1, (kc + kc_min / 2) / kc_min);
    int32_t len = (kc + ns - 1) / ns;
    len += len & 1;
    if (len >= kc) len = kc;
    out[i] = Split{(kc + len - 1) / len, len};
  }
  return out;
}

// Work units of a matrix-core grouped plan, longest unit (chunks per
// reduction range) first, so that the longest units start early and the
// launch ends on short ones.
//
// Skinny matrix-core plans large enough to fill the GPU several times are
// also ordered for the XCDs.  Consecutive workgroups go to the 8 XCDs in
// turn (workgroup i to XCD i mod 8), each with its own L2; in problem order
// every problem's tiles would spread over all 8, and each XCD would fetch
// that problem's activations from memory (measured: HBM reads 1.22 times
// the algorithmic bytes at M=32 on the 2B set, 1.25 times at M=64 on the 8B
// set).  Instead whole problems are dealt, largest first, to the XCD with
// the least work so far (each XCD's queue then runs the longest reductions
// first), and the 8 queues are interleaved so that queue x
// lands on XCD x; a queue that runs out is padded with empty units (problem
// -1, which exit at once) to keep the others aligned.  Plans in which one
// problem holds more than 1/16 of the work keep the plain order: a whole
// problem on one XCD would leave the others idle.
//
// Prefill plans of more units than compute units but at most two per unit
// (two 128-token workgroups fit a CU, so every unit is resident from the
// start: the first `cus` get a CU each and the rest double up on the CUs of
// the first ones) put the ranges of split reductions at the end of the
// first round.  Those ranges end with a combine (partials stored, counted,
// read back by the last range) that the others do not have; placed there,
// most of them run on CUs they have to themselves.  One 2B-shaped layer at
// M=512 (440 units, 120 of them ranges, on 256 CUs): 38.4-41.7 against
// 41.1-44.5 us in the plain order; the ranges first or in the second round
// were in between or slower.  Without a device the plain order stays.
constexpr int kXcds = 8;
constexpr int32_t kMaxXcdShares = 32;  // XCDs a share table may list
constexpr int64_t kXcdOrderMinUnits = 1024;
std::vector<Unit> plan_units(const bt_problem* probs, int32_t count, int m,
                             int kind, const std::vector<Split>& split,
                             int cus) {
  std::vector<int32_t> order(count);
  for (int32_t i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return split[a].len > split[b].len;
  });
  std::vector<int64_t> per(count), work(count);
  int64_t total_units = 0, total_work = 0, max_work = 0;
  for (int32_t p = 0; p < count; ++p) {
    per[p] = bt::kind_units(kind, probs[p].n, m) * split[p].nsplit;
    work[p] = per[p] * split[p].len;
    total_units += per[p];
    total_work += work[p];
    max_work = std::max(max_work, work[p]);
  }
  std::vector<Unit> units;
  if (kind != bt::kKindMfma || total_units < kXcdOrderMinUnits ||
      total_units > INT32_MAX / 64 || max_work * 16 > total_work) {
    for (int32_t p : order)
      for (int64_t s = 0; s < per[p]; ++s) units.push_back(Unit{p, (int32_t)s});
    if (kind == bt::kKindPrefill && cus > 0 && total_units > cus &&
        total_units <= 2 * (int64_t)cus) {
      std::vector<Unit> plain, ranges;
      for (const Unit& u : units)
        (split[u.prob].nsplit > 1 ? ranges : plain).push_back(u);
      if (!ranges.empty() && (int64_t)ranges.size() <= cus) {
        const size_t lead = (size_t)cus - ranges.size();  // plain units first
        std::vector<Unit> o(plain.begin(), plain.begin() + lead);
        o.insert(o.end(), ranges.begin(), ranges.end());
        o.insert(o.end(), plain.begin() + lead, plain.end());
        units.swap(o);
      }
    }
    return units;
  }
  // deal the largest problems first (for balance), then order each queue
  // longest reduction first (for the tail)
  std::vector<int32_t> by_work = order;
  std::stable_sort(by_work.begin(), by_work.end(),
                   [&](int32_t a, int32_t b) { return work[a] > work[b]; });
  std::vector<std::vector<Unit>> queue(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (int32_t p : by_work) {
    const int x = (int)(std::min_element(load.begin(), load.end()) -
                        load.begin());
    for (int64_t s = 0; s < per[p]; ++s)
      queue[x].push_back(Unit{p, (int32_t)s});
    load[x] += work[p];
  }
  for (auto& q : queue)
    std::stable_sort(q.begin(), q.end(), [&](const Unit& a, const Unit& b) {
      return split[a.prob].len > split[b.prob].len;
    });
  size_t longest = 0;
  for (const auto& q : queue) longest = std::max(longest, q.size());
  for (size_t j = 0; j < longest; ++j)
    for (int x = 0; x < kXcds; ++x)
      units.push_back(j < queue[x].size() ? queue[x][j] : Unit{-1, 0});
  return units;
}

// 1 KiB chunks of packed weights over every problem of a group.
int64_t group_chunks(const bt_problem* probs, int32_t count) {
  int64_t chunks = 0;
  for (int32_t i = 0; i < count; ++i)
    chunks += (probs[i].n + 63) / 64 * (probs[i].k / 64);
  return chunks;
}

// Plan image layout (see PlanHeader).  Offsets are 256-byte aligned.
PlanHeader plan_layout(const bt_problem* probs, int32_t count, bool fused) {
  PlanHeader h;
  memset(&h, 0, sizeof(h));
  const int m = probs[0].m;
  h.magic = bt::kPlanMagic;
  h.count = count;
  h.m = m;
  h.kind = bt::group_kind(m, group_chunks(probs, count), fused);
  const std::vector<Split> split = plan_splits(probs, count, h.kind);
  int64_t blocks = 0, chunks = 0, units = 0, slots = 0, regions = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t nblk = (probs[i].n + 63) / 64;
    blocks += nblk;
    chunks += nblk * (probs[i].k / 64);
    units += bt::kind_units(h.kind, probs[i].n, m) * split[i].nsplit;
    if (h.kind != bt::kKindDot4 && split[i].nsplit > 1) {
      const int64_t s = nblk * ((m + bt::token_tile(m) - 1) / bt::token_tile(m));
      slots += s;
      regions += s * split[i].nsplit;
    }
  }
  h.blocks = blocks;
  h.total_chunks = chunks;
  // matrix-core kinds: the unit list as built (its XCD order may pad it)
  h.units = h.kind == bt::kKindDot4
                ? units
                : (int64_t)plan_units(probs, count, m, h.kind, split, 0).size();
  // streaming kind: a start entry per wave of a launch on the current
  // device (none when no device answers)
  const int cus = h.kind == bt::kKindDot4 ? cu_count() : 0;
  h.start_waves = cus > 0 ? bt::stream_waves(chunks, cus) : 0;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  h.desc_off = up(sizeof(PlanHeader));
  h.chunk_off = up(h.desc_off + (int64_t)count * sizeof(Desc));
  h.start_off = up(h.chunk_off + (int64_t)count * 8);
  h.unit_off =
      up(h.start_off + h.start_waves * (int64_t)sizeof(bt::WaveStart));
  h.sacc_off = up(h.unit_off + h.units * (int64_t)sizeof(Unit));
  // streaming kind: one 64-bit slot (arrival count and partial total) per
  // row, token and row block; matrix-core kinds: split-reduction regions
  const int64_t sacc_bytes = h.kind == bt::kKindDot4
                                 ? blocks * m * 64 * 8
                                 : regions * bt::split_region_ints(m) * 4;
  h.scnt_off = up(h.sacc_off + sacc_bytes);
  const int64_t scnt_bytes = h.kind == bt::kKindDot4 ? 0 : slots * 4;
  h.bytes = up(h.scnt_off + scnt_bytes);
  return h;
}

int32_t check_group(const bt_problem* probs, int32_t count, bool fused) {
  if (!probs) return BT_E_NULL;
  if (count < 1 || count > (1 << 20)) return BT_E_ARG;
  int64_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    const bt_problem& p = probs[i];
    const int32_t st = check_problem(p.packed, p.s_w, p.n, p.k, p.m, p.x_q,
                                     p.s_a, p.y, p.acc);
    if (st != BT_OK) return st;
    if (p.m != probs[0].m) return BT_E_SHAPE;
    blocks += (p.n + 63) / 64;
  }
  // grid, scratch slots and unit indices stay within 32-bit ranges
  if (blocks * ((probs[0].m + 31) / 32) >= INT32_MAX / 64) return BT_E_SHAPE;
  const int kind =
      bt::group_kind(probs[0].m, group_chunks(probs, count), fused);
  if (kind != bt::kKindDot4) {
    const std::vector<Split> split = plan_splits(probs, count, kind);
    int64_t units = 0;
    for (int32_t i = 0; i < count; ++i)
      units += bt::kind_units(kind, probs[i].n, probs[i].m) * split[i].nsplit;
    // units bound the split regions (at most 4 per unit) and counters
    if (units >= INT32_MAX / 8) return BT_E_SHAPE;
  }
  return BT_OK;
}

// Header of a grouped plan, checked for consistency.
int32_t read_plan_header(const void* plan_host, PlanHeader* out) {
  PlanHeader h;
  memcpy(&h, plan_host, sizeof(h));
  if (h.magic != bt::kPlanMagic || h.count < 1 || h.blocks < 1 ||
      h.total_chunks < 1 ||
      h.m < 1 || h.m > BT_MAX_M || h.fused < 0 || h.fused > 1 ||
      h.kind != bt::group_kind(h.m, h.total_chunks, h.fused == 1) ||
      h.desc_off != 256 ||
      h.bytes < h.scnt_off || h.scnt_off < h.sacc_off ||
      h.sacc_off < h.unit_off || h.start_off < h.chunk_off + 8 * h.count ||
      h.start_waves < 0 || h.start_waves > h.total_chunks ||
      (h.start_waves > 0 && h.kind != bt::kKindDot4) ||
      h.unit_off < h.start_off + h.start_waves * (int64_t)sizeof(bt::WaveStart) ||
      h.chunk_off < h.desc_off + (int64_t)h.count * (int64_t)sizeof(Desc) ||
      (h.kind != bt::kKindDot4 && h.units < 1) ||
      (h.fused == 1 && h.kind != bt::kKindDot4) || h.sacc_off % 256 != 0 ||
      h.scnt_off % 256 != 0 || h.bytes % 256 != 0)
    return BT_E_ARG;
  *out = h;
  return BT_OK;
}

// Launches a checked plan whose descriptors are at plan_dev, with its
// scratch area (partial sums and counters) at sacc and scnt.
int32_t launch_plan(void* plan_dev, const PlanHeader& h, unsigned char* sacc,
                    unsigned char* scnt, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(plan_dev);
  const Desc* descs = reinterpret_cast<const Desc*>(base + h.desc_off);
  if (h.kind != bt::kKindDot4) {
    const Unit* units = reinterpret_cast<const Unit*>(base + h.unit_off);
    return hip_status(bt::launch_tiled_grouped(
        descs, units, h.units, h.m, reinterpret_cast<int32_t*>(sacc),
        reinterpret_cast<int32_t*>(scnt), s));
  }
  const int cus = cu_count();
  if (cus <= 0) return BT_E_HIP;
  // workgroups of 4 waves (the launch may regroup the same waves)
  const int64_t wgs = bt::stream_workgroups(h.total_chunks, cus);
  // the start table holds only if it was written for this wave count
  const bt::WaveStart* starts =
      h.start_waves > 0 && h.start_waves == bt::stream_waves(h.total_chunks, cus)
          ? reinterpret_cast<const bt::WaveStart*>(base + h.start_off)
          : nullptr;
  return hip_status(bt::launch_stream_grouped(
      descs, reinterpret_cast<const int64_t*>(base + h.chunk_off), starts,
      h.count, h.total_chunks, h.m, reinterpret_cast<int32_t*>(sacc), (int)wgs,
      h.fused == 1, wgs == (int64_t)cus * bt::kStreamWgPerCu, s));
}

// Scratch memory of bt_gemm_grouped_static: one array per GPU the library
// runs on, alive until the process ends.  In host code `scratch` is only a
// stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in g_scratch; kernels and the zero fill receive that address.
__device__ __align__(256) unsigned char scratch[BT_STATIC_SCRATCH_BYTES];
std::atomic<unsigned char*> g_scratch[kMaxDevices];

int32_t static_scratch(unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BT_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BT_E_ARCH;
  unsigned char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess ||
        addr == nullptr)
      return BT_E_HIP;
    p = static_cast<unsigned char*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return BT_OK;
}

// Host image of a chained launch: header, sync words (zeroed by every
// launch), phase table.
struct ChainHeader {
  uint32_t magic;
  int32_t count;
  int32_t m;
  int32_t pad0;
  int64_t sync_off;
  int64_t table_off;
  int64_t bytes;
  int64_t pad1[27];
};
static_assert(sizeof(ChainHeader) == 256, "ChainHeader is 256 bytes");
constexpr uint32_t kChainMagic = 0x31485442u;  // "BTH1"
constexpr int64_t kChainSyncOff = 256;
constexpr int64_t kChainTableOff =
    kChainSyncOff + (int64_t)bt::kChainSyncWords * 4;
static_assert(BT_CHAIN_STATUS_OFFSET ==
                  kChainSyncOff + 4 * (bt::kChainMaxWg + 1),
              "status word offset");

int64_t chain_bytes(int32_t count) {
  return (kChainTableOff + (int64_t)count * (int64_t)sizeof(bt::ChainPhase) +
          255) / 256 * 256;
}

// Zeroes words 16-byte words at p (vector stores; usable under graph
// capture, unlike a memset node).
__global__ __launch_bounds__(256) void zero_kernel(uint4* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Shares of the waves of a streaming launch (integers, 1000 = one equal
// share).  Equal, except on a grid that fills the GPU (8 waves per CU),
// where they follow service rates measured with per-wave timestamps (2B
// and 8B decode sets at M=1):
//  - each SIMD runs two waves, and the older one's loads go first.  With
//    8-wave workgroups (one per CU) those are waves j and j + 4 of the
//    workgroup: with equal ranges waves 4-7 took 9-13 % longer than waves
//    0-3, so they take 0.87 of a share.  With 4-wave workgroups (two per
//    CU, fused plans) the younger waves are those of the workgroups
//    dispatched second, the upper half of the grid: 0.9 of a share;
//  - workgroup g runs on XCD g mod (XCDs), and with 8 XCDs the odd ones
//    streamed 7-10 % slower on most boxes, so their workgroups take 0.9 of
//    a share.
// The waves then end together instead of the slow ones streaming on alone
// at a fraction of the bandwidth: 81 against 84.6 us on the 2B set and 262
// against 275 us on the 8B set (both weights swept over 0.82-0.92; fused
// plans 88.2 against 90.4 us and 269.9 against 276.8 us).  The outputs do
// not depend on the split.
// A caller may give its own per-XCD shares (permille, one per XCD of the
// device, from a measurement on the GPU the plan runs on): they replace the
// odd-XCD rule.
std::vector<int64_t> wave_shares(int64_t W, int wpw, bool full, int xccs,
                                 const int32_t* xcd_share = nullptr,
                                 int32_t nxcd = 0) {
  std::vector<int64_t> wt(W, 1000);
  if (!full) return wt;
  const bool own = xcd_share != nullptr && nxcd == xccs && xccs > 0;
  for (int64_t w = 0; w < W; ++w) {
    if (wpw == 8 && w % 8 >= 4) wt[w] = wt[w] * 87 / 100;
    if (wpw == 4 && w >= W / 2) wt[w] = wt[w] * 9 / 10;
    if (own)
      wt[w] = wt[w] * xcd_share[(w / wpw) % xccs] / 1000;
    else if (xccs == 8 && (w / wpw) % 2 == 1)
      wt[w] = wt[w] * 9 / 10;
  }
  return wt;
}

// Range ends by share: wave w streams chunks [b[w], b[w + 1]), b[w] =
// floor(T x (shares of waves before w) / (all shares)).
std::vector<int64_t> bounds_by_share(int64_t T,
                                     const std::vector<int64_t>& wt) {
  const int64_t W = (int64_t)wt.size();
  std::vector<int64_t> c(W + 1, 0), b(W + 1);
  for (int64_t w = 0; w < W; ++w) c[w + 1] = c[w] + wt[w];
  for (int64_t w = 0; w <= W; ++w)
    b[w] = (int64_t)((__int128)c[w] * T / c[W]);
  return b;
}

// Range ends of a launch that quantizes its own activations: every segment
// (the part of a wave's range inside one problem) starts by quantizing that
// problem's m rows, so a wave whose range crosses a problem boundary does
// that work twice.  With ranges by share, those waves finished last (per-
// wave timestamps: the fused launch's drain was 14 us on the 2B set).
// Here the ends are placed by cost instead: a chunk costs 10 units and a
// segment of problem p 4 m (k / 64) units (swept: 0.1 to 1.0 chunk per 64
// inputs of a row, best at 0.4 on both sets: 2B 84.1-84.6 against 86.8-88.0
// us, 8B 260.9-263.1 against 269.6-270.4 us; the two-launch step takes
// 85.2-85.8 and 270.9-271.1 us).  Wave w's range ends where the running cost
// first reaches C x (shares of waves up to w) / (all shares); a wave moves
// on to the next problem only if at least half of that problem's
// quantization fits its share.  C, the total cost, is set by bisection so
// that the last wave's cost matches its share.  Ranges may come out empty
// (the wave then does nothing).
constexpr int64_t kChunkCost = 10;
constexpr int64_t kQuantCostPer64 = 4;  // per 64 inputs of a token row
std::vector<int64_t> bounds_by_cost(const bt_problem* probs, int32_t count,
                                    int64_t T,
                                    const std::vector<int64_t>& wt) {
  const int64_t W = (int64_t)wt.size();
  std::vector<int64_t> ends(count), q(count), qtail(count + 1, 0);
  int64_t e = 0, qmax = 0;
  for (int32_t i = 0; i < count; ++i) {
    e += (probs[i].n + 63) / 64 * (probs[i].k / 64);
    ends[i] = e;
    q[i] = kQuantCostPer64 * probs[i].m * (probs[i].k / 64);
    qmax = std::max(qmax, q[i]);
  }
  for (int32_t i = count - 1; i >= 0; --i) qtail[i] = qtail[i + 1] + q[i];
  std::vector<int64_t> cw(W + 1, 0);
  for (int64_t w = 0; w < W; ++w) cw[w + 1] = cw[w] + wt[w];
  std::vector<int64_t> b(W + 1);
  // places the ends for total cost C; returns the last wave's cost minus
  // its share
  auto place = [&](int64_t C) -> int64_t {
    int64_t pos = 0, A = 0;
    int32_t p = 0;
    b[0] = 0;
    for (int64_t w = 0; w + 1 < W; ++w) {
      const int64_t target = (int64_t)((__int128)C * cw[w + 1] / cw[W]);
      if (pos < T) {
        while (p + 1 < count && ends[p] <= pos) ++p;
        A += q[p];  // the wave's first segment
        for (;;) {
          const int64_t left = ends[p] - pos;
          if (A + kChunkCost * left <= target && p + 1 < count) {
            A += kChunkCost * left;
            pos = ends[p];
            ++p;
            if (2 * A + q[p] > 2 * target) break;  // next wave's problem
            A += q[p];
          } else {
            const int64_t room = target - A + kChunkCost / 2;
            const int64_t step =
                std::max<int64_t>(0, std::min(left, room / kChunkCost));
            A += kChunkCost * step;
            pos += step;
            break;
          }
        }
      }
      b[w + 1] = pos;
    }
    b[W] = T;
    int64_t last = 0;
    if (pos < T) {
      while (p + 1 < count && ends[p] <= pos) ++p;
      last = qtail[p] + kChunkCost * (T - pos);
    }
    const int64_t share =
        (int64_t)((__int128)C * (cw[W] - cw[W - 1]) / cw[W]);
    return last - share;
  };
  int64_t lo = 0, hi = kChunkCost * T + W * qmax + kChunkCost;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (place(mid) > 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  place(hi);
  return b;
}

}  // namespace

extern "C" {

const char* bt_status_str(int32_t status) {
  switch (status) {
    case BT_OK: return "ok";
    case BT_E_NULL: return "a required pointer is NULL";
    case BT_E_SHAPE: return "shape out of range (need k % 64 == 0, 64 <= k <= 65536, n, m >= 1)";
    case BT_E_ALIGN: return "pointer not aligned as documented";
    case BT_E_ARG: return "invalid argument (scale, count or plan)";
    case BT_E_HIP: return "HIP runtime error";
    case BT_E_ARCH: return "current device is not gfx950";
    default: return "unknown status";
  }
}

int64_t bt_packed_bytes(int64_t n, int64_t k) {
  if (!n_ok(n) || !k_ok(k)) return BT_E_SHAPE;
  return (n + 63) / 64 * 64 * (k / 4);
}

int32_t bt_pack_i2s(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                    int32_t* n_invalid, void* stream) {
  if (!t || !packed) return BT_E_NULL;
  if (!n_ok(n) || !k_ok(k)) return BT_E_SHAPE;
  if (!aligned(t, 16) || !aligned(packed, 16) ||
      (n_invalid && !aligned(n_invalid, 4)))
    return BT_E_ALIGN;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  return hip_status(bt::launch_pack(t, n, k, packed, n_invalid,
                                    static_cast<hipStream_t>(stream)));
}

int32_t bt_quant_act(const float* x, int64_t m, int64_t k, int8_t* x_q,
                     float* s_a, void* stream) {
  if (!x || !x_q || !s_a) return BT_E_NULL;
  if (!m_ok(m) || !k_ok(k)) return BT_E_SHAPE;
  if (!aligned(x, 16) || !aligned(x_q, 16) || !aligned(s_a, 4))
    return BT_E_ALIGN;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  return hip_status(
      bt::launch_quant(x, m, k, x_q, s_a, static_cast<hipStream_t>(stream)));
}

int32_t bt_quant_act_many(const bt_quant_job* jobs, int32_t count,
                          void* stream) {
  if (!jobs) return BT_E_NULL;
  if (count < 1 || count > BT_MAX_QUANT_JOBS) return BT_E_ARG;
  int64_t rows = 0;
  for (int32_t j = 0; j < count; ++j) {
    const bt_quant_job& q = jobs[j];
    if (!q.x || !q.x_q || !q.s_a) return BT_E_NULL;
    if (!m_ok(q.m) || !k_ok(q.k)) return BT_E_SHAPE;
    if (!aligned(q.x, 16) || !aligned(q.x_q, 16) || !aligned(q.s_a, 4))
      return BT_E_ALIGN;
    rows += q.m;
  }
  if (rows > BT_MAX_M) return BT_E_SHAPE;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  return hip_status(
      bt::launch_quant_many(jobs, count, static_cast<hipStream_t>(stream)));
}

int32_t bt_gemm(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                int64_t m, const int8_t* x_q, const float* s_a, float* y,
                int32_t* acc, void* stream) {
  const int32_t st = check_problem(packed, s_w, n, k, m, x_q, s_a, y, acc);
  if (st != BT_OK) return st;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const Desc d = make_desc(packed, s_w, n, k, m, x_q, s_a, y, acc);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (bt::plan_kind(m) == bt::kKindDot4)
    return hip_status(bt::launch_dot4(d, s));
  return hip_status(bt::launch_tiled(d, s));
}

int32_t bt_gemv(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                const int8_t* x_q, const float* s_a, float* y, int32_t* acc,
                void* stream) {
  return bt_gemm(packed, s_w, n, k, 1, x_q, s_a, y, acc, stream);
}

int32_t bt_gemv_lut(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                    const int8_t* x_q, const float* s_a, float* y,
                    int32_t* acc, void* stream) {
  const int32_t st = check_problem(packed, s_w, n, k, 1, x_q, s_a, y, acc);
  if (st != BT_OK) return st;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const Desc d = make_desc(packed, s_w, n, k, 1, x_q, s_a, y, acc);
  return hip_status(bt::launch_lut(d, static_cast<hipStream_t>(stream)));
}

// Size of the plan image of a group (fused: the problems give fp32
// activations), or a negative status.
static int64_t plan_bytes_of(const bt_problem* probs, int32_t count,
                             bool fused) {
  const int32_t st = check_group(probs, count, fused);
  if (st != BT_OK) return st;
  return plan_layout(probs, count, fused).bytes;
}

int64_t bt_grouped_plan_bytes(const bt_problem* probs, int32_t count) {
  return plan_bytes_of(probs, count, false);
}

// Builds a grouped plan image; with xf, the problems give fp32 activations
// (xf[i]) that the launch quantizes itself, after an RMSNorm with gain g[i]
// and eps[i] when g is given.
static int32_t build_plan(const bt_problem* probs, int32_t count, void* plan,
                          int64_t plan_bytes, const float* const* xf,
                          const float* const* g = nullptr,
                          const float* eps = nullptr,
                          const int32_t* xcd_share = nullptr,
                          int32_t nxcd = 0) {
  if (!plan) return BT_E_NULL;
  const bool fused = xf != nullptr;
  const int32_t st = check_group(probs, count, fused);
  if (st != BT_OK) return st;
  const PlanHeader h = plan_layout(probs, count, fused);
  if (plan_bytes < h.bytes) return BT_E_ARG;
  unsigned char* out = static_cast<unsigned char*>(plan);
  memset(out, 0, (size_t)h.bytes);  // scratch area starts at zero
  PlanHeader hf = h;
  hf.fused = xf ? 1 : 0;
  memcpy(out, &hf, sizeof(hf));
  const std::vector<Split> split = plan_splits(probs, count, h.kind);
  int64_t chunk0 = 0;
  int64_t blk0 = 0;
  int64_t slot0 = 0, region0 = 0;
  for (int32_t i = 0; i < count; ++i) {
    const bt_problem& p = probs[i];
    Desc d = make_desc(p.packed, p.s_w, p.n, p.k, p.m, p.x_q, p.s_a, p.y,
                       p.acc);
    d.chunk0 = chunk0;
    d.blk0 = (int32_t)blk0;
    if (xf) {  // fused quantization: fp32 activations only
      d.xf = xf[i];
      d.xq = nullptr;
      d.sa = nullptr;
      if (g) {
        d.g = g[i];
        d.eps = eps[i];
      }
    }
    if (h.kind != bt::kKindDot4) {
      d.nsplit = split[i].nsplit;
      d.split_len = split[i].len;
      if (d.nsplit > 1) {
        d.slot0 = (int32_t)slot0;
        d.region0 = (int32_t)region0;
        slot0 += (int64_t)d.nblk * d.ntt;
        region0 += (int64_t)d.nblk * d.ntt * d.nsplit;
      }
    }
    memcpy(out + h.desc_off + (int64_t)i * sizeof(Desc), &d, sizeof(d));
    memcpy(out + h.chunk_off + (int64_t)i * 8, &chunk0, 8);
    chunk0 += (int64_t)d.nblk * d.kc;
    blk0 += d.nblk;
  }
  if (h.kind != bt::kKindDot4) {
    const std::vector<Unit> units =
        plan_units(probs, count, h.m, h.kind, split,
                   h.kind == bt::kKindPrefill ? cu_count() : 0);
    memcpy(out + h.unit_off, units.data(), units.size() * sizeof(Unit));
  }
  // start table: contiguous ranges, wave w streaming chunks [b[w], b[w+1]);
  // its first chunk lies in the last problem whose first chunk is not past
  // it
  const int64_t W = h.start_waves, T = h.total_chunks;
  const int cus = W > 0 ? cu_count() : 0;
  // a full grid has 8 waves per CU: one 8-wave workgroup per CU, or two
  // of 4 for fused plans
  const bool full = cus > 0 && W == 8 * (int64_t)cus;
  const std::vector<int64_t> wt =
      wave_shares(W, fused ? 4 : 8, full, xcc_count(), xcd_share, nxcd);
  const std::vector<int64_t> b = W <= 0 ? std::vector<int64_t>()
                                 : fused && full
                                     ? bounds_by_cost(probs, count, T, wt)
                                     : bounds_by_share(T, wt);
  int32_t p = 0;
  int64_t p0 = 0;  // first chunk of problem p
  int64_t next0 = (probs[0].n + 63) / 64 * (probs[0].k / 64);
  for (int64_t w = 0; w < W; ++w) {
    const int64_t lo = b[w];
    while (p + 1 < count && next0 <= lo) {
      ++p;
      p0 = next0;
      next0 += (probs[p].n + 63) / 64 * (probs[p].k / 64);
    }
    bt::WaveStart e;
    memset(&e, 0, sizeof(e));
    e.lo = lo;
    e.hi = b[w + 1];
    e.prev_lo = w > 0 ? b[w - 1] : 0;
    e.next_hi = w + 1 < W ? b[w + 2] : T;
    e.w = probs[p].packed;
    e.x = xf ? static_cast<const void*>(xf[p])
             : static_cast<const void*>(probs[p].x_q);
    e.chunk0 = p0;
    e.p = p;
    e.kc = (int32_t)(probs[p].k / 64);
    e.nblk = (int32_t)((probs[p].n + 63) / 64);
    memcpy(out + h.start_off + w * (int64_t)sizeof(e), &e, sizeof(e));
  }
  return BT_OK;
}

int32_t bt_grouped_plan(const bt_problem* probs, int32_t count, void* plan,
                        int64_t plan_bytes) {
  return build_plan(probs, count, plan, plan_bytes, nullptr);
}

int32_t bt_grouped_plan_xcd(const bt_problem* probs, int32_t count,
                            const int32_t* xcd_permille, int32_t nxcd,
                            void* plan, int64_t plan_bytes) {
  if (!xcd_permille) return BT_E_NULL;
  if (nxcd < 1 || nxcd > kMaxXcdShares) return BT_E_ARG;
  for (int32_t x = 0; x < nxcd; ++x)
    if (xcd_permille[x] < 500 || xcd_permille[x] > 2000) return BT_E_ARG;
  return build_plan(probs, count, plan, plan_bytes, nullptr, nullptr, nullptr,
                    xcd_permille, nxcd);
}

// The fp32-activation problems as bt_problem (x in the x_q and s_a slots,
// so that the shared checks see non-null, aligned pointers), after checks
// of their own: m <= 4 and m * k <= BT_FUSED_MAX_MK.
static int32_t as_problems(const bt_problem_f32* probs, int32_t count,
                           std::vector<bt_problem>& out) {
  if (!probs) return BT_E_NULL;
  if (count < 1 || count > (1 << 20)) return BT_E_ARG;
  out.resize(count);
  for (int32_t i = 0; i < count; ++i) {
    const bt_problem_f32& p = probs[i];
    if (!p.x) return BT_E_NULL;
    if (p.m < 1 || p.m > 4 || (int64_t)p.m * p.k > BT_FUSED_MAX_MK)
      return BT_E_SHAPE;
    out[i] = bt_problem{p.packed, reinterpret_cast<const int8_t*>(p.x), p.x,
                        p.y, p.acc, p.s_w, p.n, p.k, p.m};
  }
  return BT_OK;
}

int64_t bt_grouped_plan_f32_bytes(const bt_problem_f32* probs, int32_t count) {
  std::vector<bt_problem> q;
  const int32_t st = as_problems(probs, count, q);
  if (st != BT_OK) return st;
  return plan_bytes_of(q.data(), count, true);
}

int32_t bt_grouped_plan_f32(const bt_problem_f32* probs, int32_t count,
                            void* plan, int64_t plan_bytes) {
  std::vector<bt_problem> q;
  const int32_t st = as_problems(probs, count, q);
  if (st != BT_OK) return st;
  std::vector<const float*> xf(count);
  for (int32_t i = 0; i < count; ++i) xf[i] = probs[i].x;
  return build_plan(q.data(), count, plan, plan_bytes, xf.data());
}

// The RMSNorm problems as bt_problem_f32, after checks of their own: a
// non-null, 16-byte aligned gain and a finite, non-negative eps.
static int32_t as_problems_norm(const bt_problem_norm* probs, int32_t count,
                                std::vector<bt_problem_f32>& out) {
  if (!probs) return BT_E_NULL;
  if (count < 1 || count > (1 << 20)) return BT_E_ARG;
  out.resize(count);
  for (int32_t i = 0; i < count; ++i) {
    const bt_problem_norm& p = probs[i];
    if (!p.g) return BT_E_NULL;
    if (!aligned(p.g, 16)) return BT_E_ALIGN;
    if (!std::isfinite(p.eps) || p.eps < 0.0f) return BT_E_ARG;
    out[i] = bt_problem_f32{p.packed, p.x, p.y, p.acc, p.s_w, p.n, p.k, p.m};
  }
  return BT_OK;
}

int64_t bt_grouped_plan_norm_bytes(const bt_problem_norm* probs,
                                   int32_t count) {
  std::vector<bt_problem_f32> f;
  int32_t st = as_problems_norm(probs, count, f);
  if (st != BT_OK) return st;
  return bt_grouped_plan_f32_bytes(f.data(), count);
}

int32_t bt_grouped_plan_norm(const bt_problem_norm* probs, int32_t count,
                             void* plan, int64_t plan_bytes) {
  std::vector<bt_problem_f32> f;
  int32_t st = as_problems_norm(probs, count, f);
  if (st != BT_OK) return st;
  std::vector<bt_problem> q;
  st = as_problems(f.data(), count, q);
  if (st != BT_OK) return st;
  std::vector<const float*> xf(count), g(count);
  std::vector<float> eps(count);
  for (int32_t i = 0; i < count; ++i) {
    xf[i] = probs[i].x;
    g[i] = probs[i].g;
    eps[i] = probs[i].eps;
  }
  return build_plan(q.data(), count, plan, plan_bytes, xf.data(), g.data(),
                    eps.data());
}

int32_t bt_rmsnorm_quant(const float* x, const float* g, int64_t m, int64_t k,
                         float eps, int8_t* x_q, float* s_a, float* h,
                         void* stream) {
  if (!x || !g || !x_q || !s_a) return BT_E_NULL;
  if (!m_ok(m) || !k_ok(k)) return BT_E_SHAPE;
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(x_q, 16) ||
      !aligned(s_a, 4) || (h && !aligned(h, 16)))
    return BT_E_ALIGN;
  if (!std::isfinite(eps) || eps < 0.0f) return BT_E_ARG;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  return hip_status(bt::launch_norm_quant(x, g, m, k, eps, x_q, s_a, h,
                                          static_cast<hipStream_t>(stream)));
}

int32_t bt_gemm_grouped(void* plan_dev, const void* plan_host,
                        void* stream) {
  if (!plan_dev || !plan_host) return BT_E_NULL;
  if (!aligned(plan_dev, 256)) return BT_E_ALIGN;
  PlanHeader h;
  const int32_t st = read_plan_header(plan_host, &h);
  if (st != BT_OK) return st;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  unsigned char* base = static_cast<unsigned char*>(plan_dev);
  return launch_plan(plan_dev, h, base + h.sacc_off, base + h.scnt_off,
                     static_cast<hipStream_t>(stream));
}

int32_t bt_gemm_grouped_static(const void* plan_dev, const void* plan_host,
                               void* stream) {
  if (!plan_dev || !plan_host) return BT_E_NULL;
  if (!aligned(plan_dev, 256)) return BT_E_ALIGN;
  PlanHeader h;
  const int32_t st = read_plan_header(plan_host, &h);
  if (st != BT_OK) return st;
  // the plan's scratch area (partial sums, then counters) mapped onto the
  // static array; it must fit
  const int64_t need = h.bytes - h.sacc_off;
  if (need > BT_STATIC_SCRATCH_BYTES) return BT_E_SHAPE;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  unsigned char* scr = nullptr;
  const int32_t sst = static_scratch(&scr);
  if (sst != BT_OK) return sst;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // every launch starts from zeroed slots and counters: the array keeps
  // whatever the last call on this device left in it.  The matrix-core
  // kinds write every partial-sum region before it is read, so only their
  // counters are cleared; the streaming kind accumulates into its slots.
  const int64_t zero_from =
      h.kind == bt::kKindDot4 ? 0 : h.scnt_off - h.sacc_off;
  if (need > zero_from) {
    const int64_t words = (need - zero_from) / 16;
    zero_kernel<<<dim3((unsigned)std::min<int64_t>((words + 255) / 256, 4096)),
                  dim3(256), 0, s>>>(
        reinterpret_cast<uint4*>(scr + zero_from), words);
    if (hipGetLastError() != hipSuccess) return BT_E_HIP;
  }
  return launch_plan(const_cast<void*>(plan_dev), h, scr,
                     scr + (h.scnt_off - h.sacc_off), s);
}

int64_t bt_chain_plan_bytes(int32_t count) {
  if (count < 1 || count > BT_MAX_CHAIN_PHASES) return BT_E_ARG;
  return chain_bytes(count);
}

int32_t bt_chain_plan(const bt_chain_phase* phases, int32_t count,
                      void* chain_host, int64_t chain_bytes_given) {
  if (!phases || !chain_host) return BT_E_NULL;
  if (count < 1 || count > BT_MAX_CHAIN_PHASES) return BT_E_ARG;
  if (chain_bytes_given < chain_bytes(count)) return BT_E_ARG;
  unsigned char* out = static_cast<unsigned char*>(chain_host);
  memset(out, 0, (size_t)chain_bytes(count));
  ChainHeader ch;
  memset(&ch, 0, sizeof(ch));
  ch.magic = kChainMagic;
  ch.count = count;
  ch.sync_off = kChainSyncOff;
  ch.table_off = kChainTableOff;
  ch.bytes = chain_bytes(count);
  for (int32_t i = 0; i < count; ++i) {
    if (!phases[i].plan_dev || !phases[i].plan_host) return BT_E_NULL;
    if (!aligned(phases[i].plan_dev, 256)) return BT_E_ALIGN;
    PlanHeader h;
    const int32_t st = read_plan_header(phases[i].plan_host, &h);
    if (st != BT_OK) return st;
    // fused plans (fp32 inputs quantized in the launch), one m for all
    if (h.fused != 1 || h.kind != bt::kKindDot4) return BT_E_ARG;
    if (i == 0) ch.m = h.m;
    if (h.m != ch.m) return BT_E_SHAPE;
    unsigned char* base = static_cast<unsigned char*>(phases[i].plan_dev);
    bt::ChainPhase p;
    memset(&p, 0, sizeof(p));
    p.descs = reinterpret_cast<const Desc*>(base + h.desc_off);
    p.chunk0 = reinterpret_cast<const int64_t*>(base + h.chunk_off);
    p.sacc = reinterpret_cast<int32_t*>(base + h.sacc_off);
    p.total = h.total_chunks;
    p.count = h.count;
    memcpy(out + kChainTableOff + (int64_t)i * sizeof(p), &p, sizeof(p));
  }
  memcpy(out, &ch, sizeof(ch));
  return BT_OK;
}

int32_t bt_gemm_chain(void* chain_dev, const void* chain_host, void* stream) {
  if (!chain_dev || !chain_host) return BT_E_NULL;
  if (!aligned(chain_dev, 256)) return BT_E_ALIGN;
  ChainHeader ch;
  memcpy(&ch, chain_host, sizeof(ch));
  if (ch.magic != kChainMagic || ch.count < 1 ||
      ch.count > BT_MAX_CHAIN_PHASES || ch.m < 1 || ch.m > 4 ||
      ch.sync_off != kChainSyncOff || ch.table_off != kChainTableOff ||
      ch.bytes != chain_bytes(ch.count))
    return BT_E_ARG;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const int cus = cu_count();
  if (cus <= 0) return BT_E_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(chain_dev);
  // arrival, release and error words start at zero in every launch
  zero_kernel<<<dim3(2), dim3(256), 0, s>>>(
      reinterpret_cast<uint4*>(base + kChainSyncOff),
      (int64_t)bt::kChainSyncWords * 4 / 16);
  if (hipGetLastError() != hipSuccess) return BT_E_HIP;
  // one workgroup of 4 waves per CU, all resident (cooperative launch)
  const int wgs = std::min(cus, bt::kChainMaxWg);
  return hip_status(bt::launch_chain(
      reinterpret_cast<const bt::ChainPhase*>(base + kChainTableOff),
      ch.count, ch.m, reinterpret_cast<uint32_t*>(base + kChainSyncOff), wgs,
      s));
}

int64_t bt_b3_packed_bytes(int64_t n, int64_t k) {
  if (!n_ok(n) || !k_ok(k)) return BT_E_SHAPE;
  return bt::b3_packed_bytes(n, k);
}

int32_t bt_pack_b3(const int8_t* t, int64_t n, int64_t k, uint8_t* packed,
                   int32_t* n_invalid, void* stream) {
  if (!t || !packed) return BT_E_NULL;
  if (!n_ok(n) || !k_ok(k)) return BT_E_SHAPE;
  if (!aligned(packed, 16) || (n_invalid && !aligned(n_invalid, 4)))
    return BT_E_ALIGN;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  return hip_status(bt::launch_pack_b3(t, n, k, packed, n_invalid,
                                       static_cast<hipStream_t>(stream)));
}

int32_t bt_gemv_b3(const uint8_t* packed, float s_w, int64_t n, int64_t k,
                   const int8_t* x_q, const float* s_a, float* y, int32_t* acc,
                   void* stream) {
  const int32_t st = check_problem(packed, s_w, n, k, 1, x_q, s_a, y, acc);
  if (st != BT_OK) return st;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const Desc d = make_desc(packed, s_w, n, k, 1, x_q, s_a, y, acc);
  return hip_status(bt::launch_b3(d, static_cast<hipStream_t>(stream)));
}

int32_t bt_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                      int64_t sink_words, int32_t waves_per_cu,
                      int32_t groups, void* stream) {
  if (!buf || !sink) return BT_E_NULL;
  if (bytes < 1024 || bytes % 1024 != 0) return BT_E_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return BT_E_ALIGN;
  if ((waves_per_cu != 4 && waves_per_cu != 8) || groups < 1 || groups > 4)
    return BT_E_ARG;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const int cus = cu_count();
  if (cus <= 0) return BT_E_HIP;
  const int64_t waves = (int64_t)cus * waves_per_cu;
  if (sink_words < waves) return BT_E_SHAPE;
  return hip_status(bt::launch_read_probe(buf, bytes, sink, (int)waves,
                                          waves_per_cu, groups,
                                          static_cast<hipStream_t>(stream)));
}

int32_t bt_mix_probe(const void* buf, int64_t bytes, void* out,
                     int64_t out_bytes, int32_t burst, uint32_t* sink,
                     int64_t sink_words, int32_t waves_per_cu, int32_t groups,
                     void* stream) {
  if (!buf || !sink || (!out && out_bytes != 0)) return BT_E_NULL;
  if (bytes < 1024 || bytes % 1024 != 0 || out_bytes < 0 ||
      out_bytes % 1024 != 0 || out_bytes > bytes)
    return BT_E_SHAPE;
  if (!aligned(buf, 16) || !aligned(out, 16) || !aligned(sink, 4))
    return BT_E_ALIGN;
  if ((waves_per_cu != 4 && waves_per_cu != 8) || groups < 1 || groups > 4 ||
      burst < 1 || burst > 64)
    return BT_E_ARG;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const int cus = cu_count();
  if (cus <= 0) return BT_E_HIP;
  const int64_t waves = (int64_t)cus * waves_per_cu;
  if (sink_words < waves) return BT_E_SHAPE;
  return hip_status(bt::launch_mix_probe(
      buf, bytes, out, out_bytes, burst, sink, (int)waves, waves_per_cu,
      groups, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
