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
std::vector<Unit> plan_units(const bt_problem* probs, int32_t count, int m,
                             int kind, const std::vector<Split>& split) {
  std::vector<int32_t> order(count);
  for (int32_t i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return split[a].len > split[b].len;
  });
  std::vector<Unit> units;
  for (int32_t p : order) {
    const int64_t per = bt::kind_units(kind, probs[p].n, m) * split[p].nsplit;
    for (int64_t s = 0; s < per; ++s) units.push_back(Unit{p, (int32_t)s});
  }
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
  h.units = units;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  h.desc_off = up(sizeof(PlanHeader));
  h.chunk_off = up(h.desc_off + (int64_t)count * sizeof(Desc));
  h.unit_off = up(h.chunk_off + (int64_t)count * 8);
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
// (xf[i]) that the launch quantizes itself.
static int32_t build_plan(const bt_problem* probs, int32_t count, void* plan,
                          int64_t plan_bytes, const float* const* xf) {
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
        plan_units(probs, count, h.m, h.kind, split);
    memcpy(out + h.unit_off, units.data(), units.size() * sizeof(Unit));
  }
  return BT_OK;
}

int32_t bt_grouped_plan(const bt_problem* probs, int32_t count, void* plan,
                        int64_t plan_bytes) {
  return build_plan(probs, count, plan, plan_bytes, nullptr);
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

int32_t bt_gemm_grouped(const void* plan_dev, const void* plan_host,
                        void* stream) {
  if (!plan_dev || !plan_host) return BT_E_NULL;
  if (!aligned(plan_dev, 256)) return BT_E_ALIGN;
  PlanHeader h;
  memcpy(&h, plan_host, sizeof(h));
  if (h.magic != bt::kPlanMagic || h.count < 1 || h.blocks < 1 ||
      h.total_chunks < 1 ||
      h.m < 1 || h.m > BT_MAX_M || h.fused < 0 || h.fused > 1 ||
      h.kind != bt::group_kind(h.m, h.total_chunks, h.fused == 1) ||
      h.desc_off != 256 ||
      h.bytes < h.scnt_off || h.scnt_off < h.sacc_off ||
      h.sacc_off < h.unit_off || h.unit_off < h.chunk_off ||
      h.chunk_off < h.desc_off + (int64_t)h.count * (int64_t)sizeof(Desc) ||
      (h.kind != bt::kKindDot4 && h.units < 1) || h.fused < 0 ||
      h.fused > 1 || (h.fused == 1 && h.kind != bt::kKindDot4))
    return BT_E_ARG;
  const int32_t arch = check_arch();
  if (arch != BT_OK) return arch;
  const unsigned char* base = static_cast<const unsigned char*>(plan_dev);
  const Desc* descs = reinterpret_cast<const Desc*>(base + h.desc_off);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (h.kind != bt::kKindDot4) {
    const Unit* units = reinterpret_cast<const Unit*>(base + h.unit_off);
    unsigned char* mut = const_cast<unsigned char*>(base);
    return hip_status(bt::launch_tiled_grouped(
        descs, units, h.units, h.m, reinterpret_cast<int32_t*>(mut + h.sacc_off),
        reinterpret_cast<int32_t*>(mut + h.scnt_off), s));
  }
  const int cus = cu_count();
  if (cus <= 0) return BT_E_HIP;
  unsigned char* mut = const_cast<unsigned char*>(base);
  // at least a group of 4 chunks per wave (counted in workgroups of 4 waves;
  // the launch may regroup the same waves): a wave's set-up and hand-offs
  // cost about what streaming a few chunks does, so small plans (one phase
  // of a chained decode) run on fewer, fuller waves
  const int64_t wgs = std::min<int64_t>((int64_t)cus * bt::kStreamWgPerCu,
                                        (h.total_chunks + 15) / 16);
  return hip_status(bt::launch_stream_grouped(
      descs, reinterpret_cast<const int64_t*>(base + h.chunk_off), h.count,
      h.total_chunks, h.m, reinterpret_cast<int32_t*>(mut + h.sacc_off),
      (int)wgs, h.fused == 1, wgs == (int64_t)cus * bt::kStreamWgPerCu, s));
}

}  // extern "C"
