// C ABI of the library: argument checks, workspace layout, the per-device
// schedule-table cache, and the launch sequence of the backward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "dash_attn.h"
#include "../kernels/launch.hpp"
#include "dag.hpp"
#include "schedule.hpp"

namespace {

using dash::Sched;
using dash::Tables;

constexpr size_t kHeaderBytes = 256;   // status, work counters, XCD census (64 words)
constexpr uint32_t kDefaultSpin = 1u << 21;  // polls before giving up (seconds)
constexpr int kMaxMaskedTiles = 2048;        // tiles per side with a window or block mask

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool sched_ok(int s) { return s >= DASH_SCHED_ATOMIC && s <= DASH_SCHED_SHIFT; }
bool sched_ok_run(int s) { return sched_ok(s) || s == DASH_SCHED_AUTO; }

// Default cost model of the adaptive choice, in units of one unmasked item
// (KV tile x Q block): causal diagonal items cost half, the ordered add and
// the hand-off latency each about 5 % of an item (measured on MI355X at
// d = 128: ~24k cycles per item, ~1.2k per hand-off).
constexpr double kDefaultCost[4] = {1.0, 0.5, 0.05, 0.05};

// The ordered schedule with the smallest predicted makespan; see
// dash_schedule_choose.
dash_status choose_schedule(const dash::TileMask& m, int heads, int slots, const double cost[4],
                            Sched* choice, double pred[3]) {
  const Sched cand[3] = {Sched::Naive, Sched::Descending, Sched::Shift};
  double best = 0.0;
  int best_i = -1;
  for (int i = 0; i < 3; ++i) {
    pred[i] = NAN;
    Tables t;
    if (!dash::build_tables(m, cand[i], t)) continue;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    if (t.needs_static() && t.units() > slots) continue;
    // a subset of the heads keeps the prediction to about 2e5 items
    const long per_head = (long)t.kv.size();
    const int h = (int)std::max<long>(1, std::min<long>(heads, 200000 / std::max<long>(per_head, 1)));
    dash::DagResult r;
    if (!dash::dag_predict(t, h, slots, cost, r)) return DASH_ERR_SCHEDULE_INVALID;
    pred[i] = r.makespan;
    // ties go to the later candidate (SHIFT, then DESCENDING)
    if (best_i < 0 || r.makespan <= best) {
      best = r.makespan;
      best_i = i;
    }
  }
  if (best_i < 0) return DASH_ERR_UNSUPPORTED;
  *choice = cand[best_i];
  return DASH_OK;
}

dash_status check_desc(const dash_attn_desc* d) {
  if (!d) return DASH_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->d < 1) return DASH_ERR_INVALID_ARG;
  if (d->dtype != DASH_F32 && d->dtype != DASH_BF16) return DASH_ERR_INVALID_ARG;
  if (d->causal != 0 && d->causal != 1) return DASH_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale)) return DASH_ERR_INVALID_ARG;
  if (d->d != 64 && d->d != 128) return DASH_ERR_UNSUPPORTED;
  const int tile = d->dtype == DASH_BF16 ? 128 : 64;
  if (d->N % tile) return DASH_ERR_UNSUPPORTED;
  // row indices (head * N + row) and unit counts are 32-bit on the device
  const long long heads = (long long)d->B * d->H;
  // and byte offsets within one head's fp32 accumulator (4 * (row * d + col))
  // stay below 2^31, the out-of-range offset the kernel uses for idle loads
  if (heads * d->N >= (1LL << 31) || d->N / tile > 32767 || (long long)d->N * d->d >= (1LL << 29))
    return DASH_ERR_UNSUPPORTED;
  // mask fields
  if (d->window < 0) return DASH_ERR_INVALID_ARG;
  if (d->block_mask) {
    if (d->block_size < 1) return DASH_ERR_INVALID_ARG;
    if (d->block_size % tile || d->N % d->block_size) return DASH_ERR_UNSUPPORTED;
  }
  const bool special = d->block_mask || (d->window > 0 && d->window < d->N);
  if (special && d->N / tile > kMaxMaskedTiles) return DASH_ERR_UNSUPPORTED;
  return DASH_OK;
}

// The mask as the schedule and the kernels see it: tiles per side, causal,
// the window (0 when it covers the whole sequence) and the block mask at
// block granularity (0/1 bytes; empty without one).
struct MaskKey {
  int n = 0, tile = 0, causal = 0, window = 0, bt = 0;
  std::vector<uint8_t> block;
  bool operator<(const MaskKey& o) const {
    return std::tie(n, tile, causal, window, bt, block) <
           std::tie(o.n, o.tile, o.causal, o.window, o.bt, o.block);
  }
  bool masked() const { return causal || window > 0 || !block.empty(); }
};

MaskKey mask_key(const dash_attn_desc* d) {
  int bc = 0, br = 0;
  dash::bwd_tiles(d->dtype, d->d, &bc, &br);
  MaskKey k;
  k.tile = bc;
  k.n = d->N / bc;
  k.causal = d->causal != 0;
  k.window = (d->window > 0 && d->window < d->N) ? d->window : 0;
  if (d->block_mask) {
    k.bt = d->block_size / bc;
    const int nb = d->N / d->block_size;
    k.block.resize((size_t)nb * nb);
    for (size_t i = 0; i < k.block.size(); ++i) k.block[i] = d->block_mask[i] ? 1 : 0;
  }
  return k;
}

dash::TileMask tile_mask(const MaskKey& k) {
  return dash::make_mask(k.n, k.tile, k.causal != 0, k.window,
                         k.block.empty() ? nullptr : k.block.data(), k.bt);
}

float scale_of(const dash_attn_desc* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->d);
}

struct WsLayout {
  size_t counters_off, counters_words, acc_off, total;
};

// [0, 256): header (status word, work counter); then the order counters
// [BH, N/BR, waves]; then the fp32 dQ accumulator [BH, N, d].
WsLayout layout(const dash_attn_desc* d) {
  int bc = 0, br = 0;
  dash::bwd_tiles(d->dtype, d->d, &bc, &br);
  WsLayout w;
  const size_t heads = (size_t)d->B * d->H;
  w.counters_off = kHeaderBytes;
  w.counters_words = heads * (size_t)(d->N / br) * dash::bwd_waves(d->dtype, d->d);
  w.acc_off = align256(w.counters_off + 4 * w.counters_words);
  w.total = w.acc_off + 4 * heads * (size_t)d->N * d->d;
  return w;
}

// ----------------------------------------------------------- table cache

struct DevTables {
  Tables host;
  int* d_unit_off = nullptr;
  int2* d_items = nullptr;
};

// Per mask: tile liveness for the forward (block masks only) and the tiles
// no pair touches (their gradient rows are cleared by the host).
struct DevMask {
  dash::TileMask host;
  uint8_t* d_live = nullptr;  // [n * n] by [q * n + kv], block masks only
  int* d_dead = nullptr;      // dead Q blocks, then dead KV tiles
  int n_dead_q = 0, n_dead_kv = 0;
};

std::mutex g_mu;
std::map<std::tuple<int, MaskKey, int>, DevTables> g_tables;  // (device, mask, sched)
std::map<std::pair<int, MaskKey>, DevMask> g_masks;           // (device, mask)
std::map<std::tuple<int, int, int, int, int>, int> g_coresident;  // (device, dtype, d, masked, ordered)
std::map<std::tuple<MaskKey, int, int>, Sched> g_auto;  // (mask, heads, slots) -> choice
// (mask, sched, heads, slots, grouped) -> unit-major
std::map<std::tuple<MaskKey, int, long, int, int>, bool> g_order;

constexpr int kXcds = 8;  // XCDs of an MI355X: the group share the order choice predicts for

// Unit order of a dynamic ordered schedule: unit-major (unit 0 of every
// head, then unit 1, ...) when the DAG model predicts a makespan at least
// 5 % shorter than head by head for one group's share (the heads and
// workgroups of one XCD when units run in XCD groups).  A head's own units
// keep their relative order either way, so results are bit-identical; the
// order only changes which heads run side by side (masks whose units
// differ much in length gain most).
bool unit_major_for(const MaskKey& mkey, const Tables& t, Sched s, long heads, int maxco,
                    bool grouped) {
  if (t.needs_static() || !t.ordered() || t.units() == 0) return false;
  const auto key = std::make_tuple(mkey, (int)s, heads, maxco, (int)grouped);
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_order.find(key);
    if (it != g_order.end()) return it->second;
  }
  const int g = grouped ? kXcds : 1;
  const int slots = std::max(1, maxco / g);
  long hg = (heads + g - 1) / g;
  hg = std::max<long>(1, std::min<long>(hg, 200000 / std::max(1, t.items())));
  dash::DagResult hm, um;
  bool pick = false;
  if (dash::dag_predict(t, (int)hg, slots, kDefaultCost, hm, false) &&
      dash::dag_predict(t, (int)hg, slots, kDefaultCost, um, true))
    pick = um.makespan < 0.95 * hm.makespan;
  std::lock_guard<std::mutex> lock(g_mu);
  g_order[key] = pick;
  return pick;
}

dash_status get_mask(int dev, const MaskKey& key, const DevMask** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto mk = std::make_pair(dev, key);
  auto it = g_masks.find(mk);
  if (it != g_masks.end()) {
    *out = &it->second;
    return DASH_OK;
  }
  DevMask dm;
  dm.host = tile_mask(key);
  const int n = key.n;
  std::vector<int> dead;
  for (int q = 0; q < n; ++q) {
    bool any = false;
    for (int kv = 0; kv < n && !any; ++kv) any = dm.host.live[(size_t)q * n + kv] != 0;
    if (!any) dead.push_back(q);
  }
  dm.n_dead_q = (int)dead.size();
  for (int kv = 0; kv < n; ++kv) {
    bool any = false;
    for (int q = 0; q < n && !any; ++q) any = dm.host.live[(size_t)q * n + kv] != 0;
    if (!any) dead.push_back(kv);
  }
  dm.n_dead_kv = (int)dead.size() - dm.n_dead_q;
  if (!key.block.empty()) {
    if (hipMalloc(&dm.d_live, dm.host.live.size()) != hipSuccess) return DASH_ERR_HIP;
    if (hipMemcpy(dm.d_live, dm.host.live.data(), dm.host.live.size(), hipMemcpyHostToDevice) !=
        hipSuccess) {
      (void)hipFree(dm.d_live);
      return DASH_ERR_HIP;
    }
  }
  if (!dead.empty()) {
    if (hipMalloc(&dm.d_dead, sizeof(int) * dead.size()) != hipSuccess ||
        hipMemcpy(dm.d_dead, dead.data(), sizeof(int) * dead.size(), hipMemcpyHostToDevice) !=
            hipSuccess) {
      if (dm.d_live) (void)hipFree(dm.d_live);
      if (dm.d_dead) (void)hipFree(dm.d_dead);
      return DASH_ERR_HIP;
    }
  }
  auto res = g_masks.emplace(mk, std::move(dm));
  *out = &res.first->second;
  return DASH_OK;
}

dash_status get_tables(int dev, const MaskKey& mkey, const dash::TileMask& m, Sched s,
                       const DevTables** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto key = std::make_tuple(dev, mkey, (int)s);
  auto it = g_tables.find(key);
  if (it != g_tables.end()) {
    *out = &it->second;
    return DASH_OK;
  }
  DevTables dt;
  if (!dash::build_tables(m, s, dt.host)) return DASH_ERR_UNSUPPORTED;
  if (dash::validate_tables(dt.host)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  const Tables& t = dt.host;
  const int n = t.n;
  std::vector<int2> items(t.items());
  std::vector<int> contributors(n, 0);
  for (int i = 0; i < t.items(); ++i) ++contributors[t.q[i]];
  for (int i = 0; i < t.items(); ++i) {
    items[i].x = t.kv[i] | (t.q[i] << 16);
    // bit 29: the pair has hidden elements (the kernel masks them)
    items[i].y = t.partial[(size_t)t.q[i] * n + t.kv[i]] ? (1 << 29) : 0;
    if (t.ordered()) {
      const int r = t.rank[(size_t)t.q[i] * n + t.kv[i]];
      items[i].y |= r | ((r == contributors[t.q[i]] - 1) ? (1 << 30) : 0);
    }
  }
  if (hipMalloc(&dt.d_unit_off, sizeof(int) * t.unit_off.size()) != hipSuccess) return DASH_ERR_HIP;
  if (hipMalloc(&dt.d_items, sizeof(int2) * (items.empty() ? 1 : items.size())) != hipSuccess) {
    (void)hipFree(dt.d_unit_off);
    return DASH_ERR_HIP;
  }
  if (hipMemcpy(dt.d_unit_off, t.unit_off.data(), sizeof(int) * t.unit_off.size(),
                hipMemcpyHostToDevice) != hipSuccess ||
      (!items.empty() &&
       hipMemcpy(dt.d_items, items.data(), sizeof(int2) * items.size(), hipMemcpyHostToDevice) !=
           hipSuccess)) {
    (void)hipFree(dt.d_unit_off);
    (void)hipFree(dt.d_items);
    return DASH_ERR_HIP;
  }
  auto res = g_tables.emplace(key, std::move(dt));
  *out = &res.first->second;
  return DASH_OK;
}

dash_status get_coresident(int dev, int dtype, int d, bool masked, bool ordered, int* blocks) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto key = std::make_tuple(dev, dtype, d, (int)masked, (int)ordered);
  auto it = g_coresident.find(key);
  if (it != g_coresident.end()) {
    *blocks = it->second;
    return DASH_OK;
  }
  int b = 0;
  if (dash::bwd_max_coresident(dtype, d, masked, ordered, &b) != hipSuccess || b < 1)
    return DASH_ERR_HIP;
  g_coresident[key] = b;
  *blocks = b;
  return DASH_OK;
}

// DASH_SCHED_AUTO -> the predicted best ordered schedule for this problem
// on `maxco` co-resident workgroups (cached per shape); others unchanged.
dash_status resolve_schedule(dash_schedule schedule, const MaskKey& mkey, const dash::TileMask& m,
                             long heads, int maxco, Sched* s) {
  *s = (Sched)schedule;
  if (schedule != DASH_SCHED_AUTO) return DASH_OK;
  const int h = (int)std::min<long>(heads, 1L << 30);
  const auto key = std::make_tuple(mkey, h, maxco);
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_auto.find(key);
  if (it != g_auto.end()) {
    *s = it->second;
    return DASH_OK;
  }
  double pred[3];
  const dash_status st = choose_schedule(m, h, maxco, kDefaultCost, s, pred);
  if (st != DASH_OK) return st;
  g_auto[key] = *s;
  return DASH_OK;
}

dash_status run_bwd(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                    const void* k, const void* v, const void* dout, const float* lse,
                    const float* delta, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, const dash_bwd_debug* dbg, void* stream) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok_run(schedule)) return DASH_ERR_INVALID_ARG;
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv || !workspace)
    return DASH_ERR_INVALID_ARG;
  const WsLayout w = layout(desc);
  if (workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return DASH_ERR_WORKSPACE;
  int bc = 0, br = 0;
  dash::bwd_tiles(desc->dtype, desc->d, &bc, &br);
  const int n = desc->N / bc;
  const bool ordered = schedule != DASH_SCHED_ATOMIC;
  if (dbg && (dbg->poison_q < 0 || dbg->poison_q > desc->N / br)) return DASH_ERR_INVALID_ARG;
  if (dbg && (dbg->placement < 0 || dbg->placement > 3)) return DASH_ERR_INVALID_ARG;
  if (dbg && (dbg->unit_order < 0 || dbg->unit_order > 2)) return DASH_ERR_INVALID_ARG;
  const bool pairs = dbg && dbg->layout == 1;
  if (dbg && (dbg->layout < 0 || dbg->layout > 1)) return DASH_ERR_INVALID_ARG;
  if (pairs && (desc->dtype != 1 || desc->d != 128)) return DASH_ERR_UNSUPPORTED;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  const MaskKey mkey = mask_key(desc);
  const DevMask* dm = nullptr;
  st = get_mask(dev, mkey, &dm);
  if (st != DASH_OK) return st;
  // elements are masked inside some pairs (causal diagonal, window edges)
  const bool masked = dm->host.any_partial();
  int maxco = 0;
  st = get_coresident(dev, desc->dtype, desc->d, masked, ordered, &maxco);
  if (st != DASH_OK) return st;
  if (pairs) {
    // the wave-pair kernel must fit as many workgroups (the same schedule)
    int pb = 0;
    if (dash::bwd_pair_max_coresident(masked, ordered, &pb) != hipSuccess) return DASH_ERR_HIP;
    if (pb < maxco) return DASH_ERR_UNSUPPORTED;
  }
  const long heads = (long)desc->B * desc->H;
  Sched s = Sched::Naive;
  st = resolve_schedule(schedule, mkey, dm->host, heads, maxco, &s);
  if (st != DASH_OK) return st;
  const DevTables* tb = nullptr;
  st = get_tables(dev, mkey, dm->host, s, &tb);
  if (st != DASH_OK) return st;

  const int U = tb->host.units();
  for (int u = 0; u < U; ++u)
    if (tb->host.unit_off[u + 1] - tb->host.unit_off[u] > dash::kMaxUnitItems)
      return DASH_ERR_UNSUPPORTED;
  const long total_units = heads * U;
  int grid = 0, p_eff = 0, dynamic = 0;
  if (U == 0) {
    // no live pair at all: only the dead-tile clears below run
  } else if (tb->host.needs_static()) {
    p_eff = (maxco / U) * U;
    if (p_eff < 1) return DASH_ERR_UNSUPPORTED;  // a whole head must be resident
    if (p_eff > total_units) p_eff = (int)total_units;
    grid = p_eff;
  } else {
    dynamic = 1;
    grid = (int)std::min<long>(maxco, total_units);
    p_eff = grid;
  }

  hipStream_t strm = (hipStream_t)stream;
  char* ws = (char*)workspace;
  // ordered schedules never read an accumulator element before its first
  // contributor wrote it, so only the header and counters need clearing
  const size_t clear_bytes = ordered ? w.acc_off : w.total;
  if (dash::launch_zero_u32((uint32_t*)ws, clear_bytes / 4, strm) != hipSuccess) return DASH_ERR_HIP;

  dash::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_accum = (float*)(ws + w.acc_off);
  a.counters = (uint32_t*)(ws + w.counters_off);
  a.header = (uint32_t*)ws;
  a.unit_off = tb->d_unit_off;
  a.items = tb->d_items;
  a.N = desc->N;
  a.n_tiles = n;
  dash::mask_bounds(mkey.causal != 0, mkey.window, &a.mask_lo, &a.mask_hi);
  a.units_per_head = U;
  a.total_units = (int)total_units;
  a.p_eff = p_eff;
  a.dynamic = dynamic;
  // placement: the ordered schedules run each head on one XCD with its
  // accumulator coherent in that XCD's L2 (measured as fast or faster on
  // every workload); the atomic reference gains nothing from it
  a.xcd_mode = ordered ? 1 : 0;
  if (dbg && dbg->placement) a.xcd_mode = dbg->placement - 1;
  a.unit_major = dynamic ? (unit_major_for(mkey, tb->host, s, heads, maxco, a.xcd_mode != 0) ? 1 : 0)
                         : 0;
  if (dbg && dbg->unit_order && dynamic) a.unit_major = dbg->unit_order - 1;
  a.scale = scale_of(desc);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.spin_limit = (dbg && dbg->spin_limit) ? dbg->spin_limit : kDefaultSpin;
  a.jitter_seed = dbg ? dbg->jitter_seed : 0u;
  a.poison_q = dbg ? dbg->poison_q - 1 : -1;
  a.partials = dbg ? dbg->partials : nullptr;
  a.wait_stats = dbg ? dbg->wait_stats : nullptr;
  a.phase_stats = dbg ? dbg->phase_stats : nullptr;
  // (the wave-pair layout times 8 waves per workgroup)
  if ((a.wait_stats || a.phase_stats) &&
      (long)grid * (pairs ? 8 : dash::bwd_waves(desc->dtype, desc->d)) > 4096L * 4)
    return DASH_ERR_UNSUPPORTED;
  hipEvent_t ev0 = dbg ? (hipEvent_t)dbg->kernel_events[0] : nullptr;
  hipEvent_t ev1 = dbg ? (hipEvent_t)dbg->kernel_events[1] : nullptr;
  if (ev0 && hipEventRecord(ev0, strm) != hipSuccess) return DASH_ERR_HIP;
  if (U > 0 && (pairs ? dash::launch_bwd_pair(masked, ordered, a, grid, strm)
                       : dash::launch_bwd(desc->dtype, desc->d, masked, ordered, a, grid, strm)) !=
                   hipSuccess)
    return DASH_ERR_HIP;
  if (ev1 && hipEventRecord(ev1, strm) != hipSuccess) return DASH_ERR_HIP;
  // gradient rows no pair touches: dQ of Q blocks that see no key (the
  // atomic path's conversion already writes them), dK and dV of KV tiles no
  // query sees
  if (ordered && dm->n_dead_q &&
      dash::launch_zero_tiles(desc->dtype, dq, dm->d_dead, dm->n_dead_q, bc, desc->d, desc->N,
                              (int)heads, strm) != hipSuccess)
    return DASH_ERR_HIP;
  if (dm->n_dead_kv) {
    const int* kvs = dm->d_dead + dm->n_dead_q;
    if (dash::launch_zero_tiles(desc->dtype, dk, kvs, dm->n_dead_kv, bc, desc->d, desc->N,
                                (int)heads, strm) != hipSuccess ||
        dash::launch_zero_tiles(desc->dtype, dv, kvs, dm->n_dead_kv, bc, desc->d, desc->N,
                                (int)heads, strm) != hipSuccess)
      return DASH_ERR_HIP;
  }
  if (!ordered) {
    // the atomic schedule accumulates everything first, then scales/converts
    const size_t elems = (size_t)heads * desc->N * desc->d;
    if (dash::launch_dq_convert(desc->dtype, a.dq_accum, dq, a.scale, elems, strm) != hipSuccess)
      return DASH_ERR_HIP;
  }
  return DASH_OK;
}

}  // namespace

extern "C" {

const char* dash_status_string(dash_status s) {
  switch (s) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARG: return "invalid argument";
    case DASH_ERR_UNSUPPORTED: return "unsupported shape, dtype or schedule";
    case DASH_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DASH_ERR_HIP: return "HIP runtime error";
    case DASH_ERR_SCHEDULE_INVALID: return "schedule tables failed validation";
    case DASH_ERR_ORDER_TIMEOUT: return "ordered dQ add timed out";
  }
  return "unknown status";
}

int32_t dash_attn_tile(const dash_attn_desc* desc) {
  if (!desc) return 0;
  int bc = 0, br = 0;
  dash::bwd_tiles(desc->dtype, desc->d, &bc, &br);
  return bc;
}

int32_t dash_attn_bwd_subtile(const dash_attn_desc* desc) {
  if (!desc) return 0;
  int bc = 0, br = 0;
  dash::bwd_tiles(desc->dtype, desc->d, &bc, &br);
  return br;
}

dash_status dash_attn_fwd(const dash_attn_desc* desc, const void* q, const void* k, const void* v,
                          void* o, float* lse, void* stream) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!q || !k || !v || !o || !lse) return DASH_ERR_INVALID_ARG;
  dash::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = desc->N;
  a.BH = desc->B * desc->H;
  a.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  const MaskKey mkey = mask_key(desc);
  a.live = nullptr;
  a.n_tiles = mkey.n;
  a.tile = mkey.tile;
  dash::mask_bounds(mkey.causal != 0, mkey.window, &a.mask_lo, &a.mask_hi);
  if (!mkey.block.empty()) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
    const DevMask* dm = nullptr;
    st = get_mask(dev, mkey, &dm);
    if (st != DASH_OK) return st;
    a.live = dm->d_live;
  }
  if (dash::launch_fwd(desc->dtype, desc->d, mkey.masked(), a, (hipStream_t)stream) != hipSuccess)
    return DASH_ERR_HIP;
  return DASH_OK;
}

dash_status dash_attn_bwd_preprocess(const dash_attn_desc* desc, const void* o, const void* dout,
                                     float* delta, void* stream) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!o || !dout || !delta) return DASH_ERR_INVALID_ARG;
  const long rows = (long)desc->B * desc->H * desc->N;
  if (dash::launch_preprocess(desc->dtype, desc->d, o, dout, delta, rows, (hipStream_t)stream) !=
      hipSuccess)
    return DASH_ERR_HIP;
  return DASH_OK;
}

dash_status dash_attn_bwd_workspace_size(const dash_attn_desc* desc, dash_schedule schedule,
                                         size_t* bytes) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok_run(schedule) || !bytes) return DASH_ERR_INVALID_ARG;
  *bytes = layout(desc).total;
  return DASH_OK;
}

dash_status dash_attn_bwd(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                          const void* k, const void* v, const void* dout, const float* lse,
                          const float* delta, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run_bwd(desc, schedule, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                 workspace_bytes, nullptr, stream);
}

dash_status dash_attn_bwd_debug(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                                const void* k, const void* v, const void* dout, const float* lse,
                                const float* delta, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, const dash_bwd_debug* dbg, void* stream) {
  if (!dbg) return DASH_ERR_INVALID_ARG;
  return run_bwd(desc, schedule, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                 workspace_bytes, dbg, stream);
}

dash_status dash_attn_bwd_tune(const dash_attn_desc* desc, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, int32_t reps, dash_schedule* choice,
                              float* times_ms, void* stream) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (reps < 1 || reps > 1000 || !choice) return DASH_ERR_INVALID_ARG;
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv || !workspace)
    return DASH_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  const MaskKey mkey = mask_key(desc);
  const DevMask* dm = nullptr;
  st = get_mask(dev, mkey, &dm);
  if (st != DASH_OK) return st;
  int maxco = 0;
  st = get_coresident(dev, desc->dtype, desc->d, dm->host.any_partial(), true, &maxco);
  if (st != DASH_OK) return st;
  hipStream_t strm = (hipStream_t)stream;
  hipEvent_t ev[2];
  if (hipEventCreate(&ev[0]) != hipSuccess) return DASH_ERR_HIP;
  if (hipEventCreate(&ev[1]) != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return DASH_ERR_HIP;
  }
  const dash_schedule cand[3] = {DASH_SCHED_NAIVE, DASH_SCHED_DESCENDING, DASH_SCHED_SHIFT};
  float t[3];
  int best = -1;
  for (int i = 0; i < 3 && st == DASH_OK; ++i) {
    t[i] = NAN;
    Tables tb;
    if (!dash::build_tables(dm->host, (Sched)cand[i], tb)) continue;
    if (tb.needs_static() && tb.units() > maxco) continue;
    // one untimed launch, then `reps` timed ones
    st = run_bwd(desc, cand[i], q, k, v, dout, lse, delta, dq, dk, dv, workspace, workspace_bytes,
                 nullptr, stream);
    if (st == DASH_ERR_UNSUPPORTED) {  // e.g. a unit longer than the kernel's work list
      st = DASH_OK;
      continue;
    }
    if (st != DASH_OK) break;
    if (hipEventRecord(ev[0], strm) != hipSuccess) st = DASH_ERR_HIP;
    for (int r = 0; r < reps && st == DASH_OK; ++r)
      st = run_bwd(desc, cand[i], q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                   workspace_bytes, nullptr, stream);
    if (st != DASH_OK) break;
    if (hipEventRecord(ev[1], strm) != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess) {
      st = DASH_ERR_HIP;
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) {
      st = DASH_ERR_HIP;
      break;
    }
    t[i] = ms / reps;
    if (best < 0 || t[i] < t[best]) best = i;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (st != DASH_OK) return st;
  // a time-out of an ordered add would make the times meaningless
  st = dash_attn_bwd_status(workspace, stream);
  if (st != DASH_OK) return st;
  if (best < 0) return DASH_ERR_UNSUPPORTED;
  {
    const int h = (int)std::min<long>((long)desc->B * desc->H, 1L << 30);
    std::lock_guard<std::mutex> lock(g_mu);
    g_auto[std::make_tuple(mkey, h, maxco)] = (Sched)cand[best];
  }
  *choice = cand[best];
  if (times_ms) std::memcpy(times_ms, t, sizeof(t));
  return DASH_OK;
}

dash_status dash_attn_bwd_status(const void* workspace, void* stream) {
  if (!workspace) return DASH_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DASH_ERR_HIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return DASH_ERR_HIP;
  return word ? DASH_ERR_ORDER_TIMEOUT : DASH_OK;
}

dash_status dash_schedule_tables(int32_t n, int32_t causal, dash_schedule schedule,
                                 int32_t* n_units, int32_t* unit_offsets, int32_t* item_kv,
                                 int32_t* item_q, int32_t* rank) {
  if (n < 1 || n > 32767 || (causal != 0 && causal != 1) || !sched_ok(schedule) || !n_units ||
      !unit_offsets || !item_kv || !item_q || !rank)
    return DASH_ERR_INVALID_ARG;
  Tables t;
  if (!dash::build_tables(n, causal != 0, (Sched)schedule, t)) return DASH_ERR_UNSUPPORTED;
  if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  *n_units = t.units();
  std::memcpy(unit_offsets, t.unit_off.data(), sizeof(int) * t.unit_off.size());
  std::memcpy(item_kv, t.kv.data(), sizeof(int) * t.kv.size());
  std::memcpy(item_q, t.q.data(), sizeof(int) * t.q.size());
  std::memcpy(rank, t.rank.data(), sizeof(int) * t.rank.size());
  return DASH_OK;
}

dash_status dash_schedule_predict(int32_t n, int32_t causal, dash_schedule schedule, int32_t heads,
                                  int32_t slots, const double cost[4], double out[4]) {
  if (n < 1 || n > 32767 || (causal != 0 && causal != 1) || !sched_ok(schedule) || heads < 1 ||
      slots < 1 || !cost || !out)
    return DASH_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!(cost[i] >= 0.0) || !std::isfinite(cost[i])) return DASH_ERR_INVALID_ARG;
  Tables t;
  if (!dash::build_tables(n, causal != 0, (Sched)schedule, t)) return DASH_ERR_UNSUPPORTED;
  if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  if (t.needs_static() && t.units() > slots) return DASH_ERR_UNSUPPORTED;
  dash::DagResult r;
  if (!dash::dag_predict(t, heads, slots, cost, r)) return DASH_ERR_SCHEDULE_INVALID;
  out[0] = r.makespan;
  out[1] = r.total_wait;
  out[2] = r.max_slot_idle;
  out[3] = r.lower_bound;
  return DASH_OK;
}

dash_status dash_attn_bwd_resolve_schedule(const dash_attn_desc* desc, dash_schedule schedule,
                                           dash_schedule* resolved) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok_run(schedule) || !resolved) return DASH_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  const MaskKey mkey = mask_key(desc);
  const DevMask* dm = nullptr;
  st = get_mask(dev, mkey, &dm);
  if (st != DASH_OK) return st;
  int maxco = 0;
  st = get_coresident(dev, desc->dtype, desc->d, dm->host.any_partial(),
                      schedule != DASH_SCHED_ATOMIC, &maxco);
  if (st != DASH_OK) return st;
  Sched s = Sched::Naive;
  st = resolve_schedule(schedule, mkey, dm->host, (long)desc->B * desc->H, maxco, &s);
  if (st != DASH_OK) return st;
  *resolved = (dash_schedule)s;
  return DASH_OK;
}

dash_status dash_schedule_choose(int32_t n, int32_t causal, int32_t heads, int32_t slots,
                                 const double* cost, dash_schedule* choice, double* predicted) {
  if (n < 1 || n > 32767 || (causal != 0 && causal != 1) || heads < 1 || slots < 1 || !choice)
    return DASH_ERR_INVALID_ARG;
  const double* c = cost ? cost : kDefaultCost;
  for (int i = 0; i < 4; ++i)
    if (!(c[i] >= 0.0) || !std::isfinite(c[i])) return DASH_ERR_INVALID_ARG;
  Sched s = Sched::Naive;
  double pred[3];
  const dash_status st = choose_schedule(dash::plain_mask(n, causal != 0), heads, slots, c, &s, pred);
  if (st != DASH_OK) return st;
  *choice = (dash_schedule)s;
  if (predicted) std::memcpy(predicted, pred, sizeof(pred));
  return DASH_OK;
}

dash_status dash_attn_schedule_tables(const dash_attn_desc* desc, dash_schedule schedule,
                                      int32_t sizes[4], int32_t* unit_offsets, int32_t* item_kv,
                                      int32_t* item_q, int32_t* item_step, uint8_t* item_partial,
                                      int32_t* rank) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok(schedule) || !sizes) return DASH_ERR_INVALID_ARG;
  const MaskKey mkey = mask_key(desc);
  const dash::TileMask m = tile_mask(mkey);
  Tables t;
  if (!dash::build_tables(m, (Sched)schedule, t)) return DASH_ERR_UNSUPPORTED;
  if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  const bool fill = unit_offsets && item_kv && item_q && item_step && item_partial && rank;
  if (fill && (sizes[0] != t.n || sizes[1] != t.units() || sizes[2] != t.items()))
    return DASH_ERR_INVALID_ARG;
  sizes[0] = t.n;
  sizes[1] = t.units();
  sizes[2] = t.items();
  sizes[3] = t.needs_static() ? 1 : 0;
  if (!fill) return DASH_OK;
  std::memcpy(unit_offsets, t.unit_off.data(), sizeof(int) * t.unit_off.size());
  if (t.items()) {
    std::memcpy(item_kv, t.kv.data(), sizeof(int) * t.kv.size());
    std::memcpy(item_q, t.q.data(), sizeof(int) * t.q.size());
  }
  for (int i = 0; i < t.items(); ++i) {
    item_step[i] = t.step.empty() ? -1 : t.step[i];
    item_partial[i] = t.partial[(size_t)t.q[i] * t.n + t.kv[i]];
  }
  std::memcpy(rank, t.rank.data(), sizeof(int) * t.rank.size());
  return DASH_OK;
}

dash_status dash_attn_schedule_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                       int32_t slots, int32_t unit_major, const double cost[4],
                                       double out[4]) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok(schedule) || slots < 1 || !cost || !out || (unit_major != 0 && unit_major != 1))
    return DASH_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!(cost[i] >= 0.0) || !std::isfinite(cost[i])) return DASH_ERR_INVALID_ARG;
  Tables t;
  if (!dash::build_tables(tile_mask(mask_key(desc)), (Sched)schedule, t)) return DASH_ERR_UNSUPPORTED;
  if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  if (t.needs_static() && t.units() > slots) return DASH_ERR_UNSUPPORTED;
  dash::DagResult r;
  if (!dash::dag_predict(t, desc->B * desc->H, slots, cost, r, unit_major != 0))
    return DASH_ERR_SCHEDULE_INVALID;
  out[0] = r.makespan;
  out[1] = r.total_wait;
  out[2] = r.max_slot_idle;
  out[3] = r.lower_bound;
  return DASH_OK;
}

dash_status dash_dag_longest_path(int32_t n_nodes, const double* weights, int32_t n_edges,
                                  const int32_t* src, const int32_t* dst, const double* latency,
                                  double* start, double* finish) {
  if (n_nodes < 0 || n_edges < 0 || (n_nodes && (!weights || !start || !finish)) ||
      (n_edges && (!src || !dst || !latency)))
    return DASH_ERR_INVALID_ARG;
  for (int e = 0; e < n_edges; ++e)
    if (src[e] < 0 || src[e] >= n_nodes || dst[e] < 0 || dst[e] >= n_nodes)
      return DASH_ERR_INVALID_ARG;
  if (!dash::dag_longest_path(n_nodes, weights, n_edges, src, dst, latency, start, finish))
    return DASH_ERR_SCHEDULE_INVALID;
  return DASH_OK;
}

dash_status dash_litmus_ordered_add(int32_t workgroups, int32_t len, const int32_t* turn,
                                    const float* values, float* acc, uint32_t* counters,
                                    uint32_t spin_limit, void* stream) {
  if (workgroups < 1 || len < 1 || !turn || !values || !acc || !counters)
    return DASH_ERR_INVALID_ARG;
  hipStream_t strm = (hipStream_t)stream;
  if (dash::launch_zero_u32(counters, 2, strm) != hipSuccess) return DASH_ERR_HIP;
  if (dash::launch_litmus(workgroups, len, turn, values, acc, counters, counters + 1,
                          spin_limit ? spin_limit : kDefaultSpin, strm) != hipSuccess)
    return DASH_ERR_HIP;
  if (hipStreamSynchronize(strm) != hipSuccess) return DASH_ERR_HIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, counters + 1, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return DASH_ERR_HIP;
  return word ? DASH_ERR_ORDER_TIMEOUT : DASH_OK;
}

}  // extern "C"
