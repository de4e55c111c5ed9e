// C ABI of the library: argument checks, workspace layout, the host-side
// schedule-table cache, and the launch sequence of the backward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "dash_attn.h"
#include "../kernels/launch.hpp"
#include "../kernels/plain_tables.hpp"
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
// The two-stage pipeline layout overlaps a sub-tile's products with the
// previous sub-tile's dQ add, so an item costs less and the chain of ordered
// adds relatively more: fitted to its times on MI355X (the add and the
// hand-off each about 30 % of an item; this model picks the fastest ordered
// schedule on the causal, full, sliding-window and block-sparse workloads).
constexpr double kPipeCost[4] = {1.0, 0.5, 0.3, 0.3};
typedef std::array<double, 4> Cost;

// Backward kernel layouts (dash_bwd_debug.layout): 0 automatic, 1 wave
// pairs, 2 two-stage pipeline, 3 one-stage kernel.
constexpr int kLayoutPairs = 1, kLayoutPipe = 2, kLayoutOneStage = 3;
// The layout an automatic launch runs: the pipeline where it exists (bf16,
// d = 128 or 64), else the one-stage kernel.
int auto_layout(int dtype, int d) {
  return dtype == DASH_BF16 && (d == 128 || d == 64) ? kLayoutPipe : kLayoutOneStage;
}

constexpr int kXcds = 8;  // XCDs of an MI355X: the workgroup groups of the placement

// How a launch runs a schedule's tables, as the kernel places them: the
// ordered schedules run in XCD groups (each group's workgroups take the units
// of 1/8 of the heads) unless a static table's units do not fit one group's
// workgroups (then device-wide); the dynamic tables take units head by head,
// or unit-major when that is predicted at least 5 % shorter.
struct LaunchPrediction {
  dash::DagResult r;   // makespan etc. of one group's share (all groups alike)
  int groups = 1;      // 8 (XCD groups) or 1 (device-wide)
  int unit_major = 0;  // the dynamic unit order
  int heads = 0, slots = 0;  // the share the model ran (sampled when large)
};

// DAG prediction of a launch on `maxco` co-resident workgroups (grouped:
// whether the launch places units in XCD groups when they fit).  A group's
// share larger than about 2e5 items is sampled: fewer heads on the same
// workgroups (whole rounds for static tables), the times scaled up by the
// ratio of heads (steady state: each further head adds the same work).
bool launch_predict(const Tables& t, long heads, int maxco, const double cost[4], bool grouped,
                    LaunchPrediction& out) {
  if (heads < 1 || maxco < 1) return false;
  if (t.units() == 0) {  // every pair masked: nothing runs
    out = LaunchPrediction();
    out.slots = maxco;
    return true;
  }
  int g = grouped ? kXcds : 1;
  if (maxco / g < 1 || (t.needs_static() && t.units() > maxco / g)) g = 1;
  if (t.needs_static() && t.units() > maxco) return false;
  const int slots = maxco / g;
  const long hg = (heads + g - 1) / g;
  long hs = hg;
  const long cap = std::max<long>(1, 200000 / std::max(1, t.items()));
  if (hs > cap) {
    hs = cap;
    if (t.needs_static()) {
      const long per_round = slots / t.units();  // heads of one round
      hs = std::max(per_round, (hs / per_round) * per_round);
    }
  }
  out.groups = g;
  out.heads = (int)hs;
  out.slots = slots;
  out.unit_major = 0;
  if (!dash::dag_predict(t, (int)hs, slots, cost, out.r, false)) return false;
  if (!t.needs_static() && t.ordered()) {
    dash::DagResult um;
    if (dash::dag_predict(t, (int)hs, slots, cost, um, true) &&
        um.makespan < 0.95 * out.r.makespan) {
      out.r = um;
      out.unit_major = 1;
    }
  }
  if (hs < hg) {
    const double f = (double)hg / (double)hs;
    out.r.makespan *= f;
    out.r.total_wait *= f;
    out.r.max_slot_idle *= f;
    out.r.lower_bound *= f;
  }
  return true;
}

// The tables a launch on `slots` co-resident workgroups runs for `heads`
// heads (the timed shift of a special mask depends on both).  Returns false
// where the schedule is undefined.
bool launch_tables(const dash::TileMask& m, Sched s, long heads, int slots, Tables& t) {
  int ws = 1;
  if (!m.plain) {
    int live_kv = 0;
    for (int kv = 0; kv < m.n; ++kv)
      for (int q = 0; q < m.n; ++q)
        if (m.live[(size_t)q * m.n + kv]) {
          ++live_kv;
          break;
        }
    ws = dash::timed_slots(slots, heads, live_kv);
  }
  return dash::build_tables(m, s, t, ws);
}

// The ordered schedule with the smallest predicted makespan; see
// dash_schedule_choose.  placement: predict each schedule as the launch
// places it (launch_predict, on `slots` co-resident workgroups); otherwise
// all `heads` heads head by head on `slots` workgroups.
dash_status choose_schedule(const dash::TileMask& m, int heads, int slots, const double cost[4],
                            Sched* choice, double pred[3], bool placement = false) {
  const Sched cand[3] = {Sched::Naive, Sched::Descending, Sched::Shift};
  double best = 0.0;
  int best_i = -1;
  for (int i = 0; i < 3; ++i) {
    pred[i] = NAN;
    Tables t;
    if (!launch_tables(m, cand[i], heads, slots, t)) continue;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    if (t.needs_static() && t.units() > slots) continue;
    dash::DagResult r;
    if (placement) {
      LaunchPrediction lp;
      if (!launch_predict(t, heads, slots, cost, true, lp)) return DASH_ERR_SCHEDULE_INVALID;
      r = lp.r;
    } else {
      // a subset of the heads keeps the prediction to about 2e5 items
      const long per_head = (long)t.kv.size();
      const int h =
          (int)std::max<long>(1, std::min<long>(heads, 200000 / std::max<long>(per_head, 1)));
      if (!dash::dag_predict(t, h, slots, cost, r)) return DASH_ERR_SCHEDULE_INVALID;
    }
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

// The DAG model's costs fitted to measured kernel times ms[3] of NAIVE,
// DESCENDING and SHIFT (NaN or <= 0: not measured; at least two needed), each
// predicted as a launch on `slots` co-resident workgroups places it: c_full
// = 1, c_diag, r and h on a grid, and per candidate the time of one item
// unit that best matches all measured times (least squares on relative
// error).  The candidate with the smallest relative RMS error wins; ties go
// to the one nearest the defaults.  Host only.
dash_status fit_costs(const dash::TileMask& m, long heads, int slots, const double ms[3],
                      Cost& out, double* residual, double* item_ms) {
  const Sched cand[3] = {Sched::Naive, Sched::Descending, Sched::Shift};
  std::vector<Tables> tabs;
  std::vector<double> meas;
  for (int i = 0; i < 3; ++i) {
    if (!(ms[i] > 0.0) || !std::isfinite(ms[i])) continue;
    Tables t;
    if (!launch_tables(m, cand[i], heads, slots, t)) return DASH_ERR_UNSUPPORTED;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    if (t.needs_static() && t.units() > slots) return DASH_ERR_UNSUPPORTED;
    if (t.units() == 0) return DASH_ERR_UNSUPPORTED;  // nothing runs: nothing to fit
    tabs.push_back(std::move(t));
    meas.push_back(ms[i]);
  }
  if (tabs.size() < 2) return DASH_ERR_INVALID_ARG;
  const double cd_grid[] = {0.5, 0.75, 1.0};
  const double rh_grid[] = {0.0, 0.025, 0.05, 0.1, 0.2, 0.3};
  double best = INFINITY, best_dist = INFINITY, best_scale = 0.0;
  for (double cd : cd_grid)
    for (double r : rh_grid)
      for (double h : rh_grid) {
        const double cost[4] = {1.0, cd, r, h};
        // a_i = predicted / measured; scale t minimises sum (t a_i - 1)^2
        double sa = 0.0, saa = 0.0;
        std::vector<double> a;
        for (size_t i = 0; i < tabs.size(); ++i) {
          LaunchPrediction lp;
          if (!launch_predict(tabs[i], heads, slots, cost, true, lp)) return DASH_ERR_SCHEDULE_INVALID;
          a.push_back(lp.r.makespan / meas[i]);
          sa += a.back();
          saa += a.back() * a.back();
        }
        if (!(saa > 0.0)) continue;
        const double tsc = sa / saa;
        double err = 0.0;
        for (double ai : a) err += (tsc * ai - 1.0) * (tsc * ai - 1.0);
        err = std::sqrt(err / (double)a.size());
        const double dist = std::fabs(cd - kDefaultCost[1]) + std::fabs(r - kDefaultCost[2]) +
                            std::fabs(h - kDefaultCost[3]);
        if (err < best - 1e-12 || (err <= best + 1e-12 && dist < best_dist)) {
          best = err;
          best_dist = dist;
          best_scale = tsc;
          out = Cost{1.0, cd, r, h};
        }
      }
  if (!std::isfinite(best)) return DASH_ERR_UNSUPPORTED;
  if (residual) *residual = best;
  if (item_ms) *item_ms = best_scale;  // measured time per cost unit
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

// ----------------------------------------------------------- workspace

// [0, 256): header (status word, work counters, XCD census); the order
// counters [BH, N/BR, waves] u32; one head's schedule tables (unit offsets
// [n + 1], items [live pairs] int2, and the Q blocks / KV tiles no pair
// touches [<= 2n]); the fp32 dQ accumulator [BH, N, d].  The table region
// holds the largest table any schedule builds for the mask (at most n + 1
// units, one item per live pair), so the size is the same for every
// schedule.
struct WsLayout {
  size_t counters_off, counters_words, unit_off_off, items_off, dead_off, lse2_off, acc_off, total;
};

WsLayout layout(const dash_attn_desc* d, long live_pairs) {
  int bc = 0, br = 0;
  dash::bwd_tiles(d->dtype, d->d, &bc, &br);
  const int n = d->N / bc;
  WsLayout w;
  const size_t heads = (size_t)d->B * d->H;
  w.counters_off = kHeaderBytes;
  w.counters_words = heads * (size_t)(d->N / br) * dash::bwd_waves(d->dtype, d->d);
  w.unit_off_off = align256(w.counters_off + 4 * w.counters_words);
  w.items_off = align256(w.unit_off_off + 4 * (size_t)(n + 1));
  w.dead_off = align256(w.items_off + 8 * (size_t)std::max<long>(live_pairs, 1));
  w.lse2_off = align256(w.dead_off + 4 * (size_t)(2 * n));
  w.acc_off = align256(w.lse2_off + 4 * heads * (size_t)d->N);
  w.total = w.acc_off + 4 * heads * (size_t)d->N * d->d;
  return w;
}

bool plain_key(const MaskKey& k) { return k.window == 0 && k.block.empty(); }

// ------------------------------------------------------ host table caches
//
// Host memory only.  Plain masks: the host builds and validates the tables
// once and checks them against the closed forms the device writes into the
// workspace at every launch.  Windows and block masks: the host builds the
// tables and keeps them in pinned host memory, laid out as the workspace's
// table region, and every launch copies them into the caller's workspace on
// the caller's stream.  Entries are evicted least recently used beyond
// kMaxEntries; an evicted pinned buffer is freed only after the last copy
// from it has completed (an event recorded behind each copy).

constexpr size_t kMaxEntries = 32;

struct MaskEntry {
  dash::TileMask host;
  long live_pairs = 0;
  std::vector<int> dead;  // Q blocks no pair touches, then KV tiles
  int n_dead_q = 0, n_dead_kv = 0;
  uint8_t* pinned_live = nullptr;  // block masks: tile liveness for the forward
  hipEvent_t used = nullptr;
  uint64_t stamp = 0;
};

struct TabEntry {
  Tables host;
  int max_unit_items = 0;
  char* pinned = nullptr;  // special masks: unit offsets | items | dead list
  size_t bytes = 0;
  hipEvent_t used = nullptr;
  uint64_t stamp = 0;
};

std::mutex g_mu;
uint64_t g_clock = 0;
std::map<MaskKey, MaskEntry> g_masks;                     // special masks only
std::map<std::tuple<MaskKey, int, int>, TabEntry> g_tables;  // (mask, sched, timed slots)
std::map<std::tuple<int, int, int, int, int>, int> g_coresident;  // (device, dtype, d, masked, ordered)
// AUTO: the problem on a device (device, dtype, d, mask, heads, co-resident
// workgroups); its model pick is cached per cost vector, a pick that
// dash_attn_bwd_tune measured takes precedence
typedef std::tuple<int, int, int, MaskKey, int, int> AutoKey;
std::map<std::pair<AutoKey, Cost>, Sched> g_auto;
std::map<AutoKey, Sched> g_tuned;
// costs AUTO uses per (device, dtype, d) once dash_attn_bwd_calibrate fitted them
std::map<std::tuple<int, int, int>, Cost> g_costs;
// (mask, sched, heads, slots, grouped, costs) -> unit-major
std::map<std::tuple<MaskKey, int, long, int, int, Cost>, bool> g_order;

template <typename E>
void release_entry(E& e, void* buf) {
  if (e.used) {
    (void)hipEventSynchronize(e.used);
    (void)hipEventDestroy(e.used);
    e.used = nullptr;
  }
  if (buf) (void)hipHostFree(buf);
}

void free_entry(MaskEntry& e) { release_entry(e, e.pinned_live); e.pinned_live = nullptr; }
void free_entry(TabEntry& e) { release_entry(e, e.pinned); e.pinned = nullptr; }

template <typename M>
void evict(M& m) {
  while (m.size() >= kMaxEntries) {
    auto victim = m.begin();
    for (auto it = m.begin(); it != m.end(); ++it)
      if (it->second.stamp < victim->second.stamp) victim = it;
    free_entry(victim->second);
    m.erase(victim);
  }
}

// The mask entry of a window or block mask (caller holds g_mu).
MaskEntry* mask_entry(const MaskKey& key) {
  auto it = g_masks.find(key);
  if (it != g_masks.end()) {
    it->second.stamp = ++g_clock;
    return &it->second;
  }
  evict(g_masks);
  MaskEntry e;
  e.host = tile_mask(key);
  const int n = key.n;
  for (int q = 0; q < n; ++q) {
    bool any = false;
    for (int kv = 0; kv < n; ++kv) {
      const bool l = e.host.live[(size_t)q * n + kv] != 0;
      any = any || l;
      e.live_pairs += l ? 1 : 0;
    }
    if (!any) e.dead.push_back(q);
  }
  e.n_dead_q = (int)e.dead.size();
  for (int kv = 0; kv < n; ++kv) {
    bool any = false;
    for (int q = 0; q < n && !any; ++q) any = e.host.live[(size_t)q * n + kv] != 0;
    if (!any) e.dead.push_back(kv);
  }
  e.n_dead_kv = (int)e.dead.size() - e.n_dead_q;
  e.stamp = ++g_clock;
  return &g_masks.emplace(key, std::move(e)).first->second;
}

// Live tile pairs of a descriptor's mask (caller holds g_mu for special masks).
long live_pairs_of(const MaskKey& key) {
  if (plain_key(key)) return dash::plain::items(key.n, key.causal != 0);
  return mask_entry(key)->live_pairs;
}

std::vector<int2> encode_items(const Tables& t) {
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
  return items;
}

// Most items of one unit of a plain schedule (without building it).
int plain_max_unit_items(int n, bool causal, Sched s) {
  return (s == Sched::Shift && causal && n > 1) ? n + 1 : n;
}

// Slots per head of the timed shift that a launch on `maxco` co-resident
// workgroups runs for a window or block mask (0: other schedules and the
// plain masks, whose tables do not depend on it).  Caller holds g_mu.
int plan_slots(const MaskKey& key, Sched s, long heads, int maxco) {
  if (s != Sched::Shift || plain_key(key)) return 0;
  return dash::timed_slots(maxco, heads, key.n - mask_entry(key)->n_dead_kv);
}

// Tables of (mask, schedule, timed slots from plan_slots), built, validated
// and (plain masks) checked against the closed forms the device writes.
// Host memory only.  Caller holds g_mu.
dash_status tab_entry(const MaskKey& key, Sched s, int ws, TabEntry** out) {
  const auto k = std::make_tuple(key, (int)s, ws);
  auto it = g_tables.find(k);
  if (it != g_tables.end()) {
    it->second.stamp = ++g_clock;
    *out = &it->second;
    return DASH_OK;
  }
  const bool plain = plain_key(key);
  const int n = key.n;
  if (plain && plain_max_unit_items(n, key.causal != 0, s) > dash::kMaxUnitItems)
    return DASH_ERR_UNSUPPORTED;
  TabEntry e;
  if (plain) {
    if (!dash::build_tables(n, key.causal != 0, s, e.host)) return DASH_ERR_UNSUPPORTED;
  } else {
    if (!dash::build_tables(mask_entry(key)->host, s, e.host, ws > 0 ? ws : 1))
      return DASH_ERR_UNSUPPORTED;
  }
  const Tables& t = e.host;
  if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
  for (int u = 0; u < t.units(); ++u)
    e.max_unit_items = std::max(e.max_unit_items, t.unit_off[u + 1] - t.unit_off[u]);
  if (e.max_unit_items > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
  if (plain) {
    // the device writes the closed forms: they must be these tables
    const std::vector<int2> items = encode_items(t);
    const bool c = key.causal != 0;
    const int ps = (int)s;
    bool same = dash::plain::defined(n, c, ps) && dash::plain::units(n, c, ps) == t.units() &&
                dash::plain::items(n, c) == (long)t.items();
    for (int u = 0; same && u <= t.units(); ++u)
      same = dash::plain::unit_off(n, c, ps, u) == (long)t.unit_off[u];
    for (int i = 0; same && i < t.items(); ++i) {
      const int2 g = dash::plain::encode(n, c, ps, i);
      same = g.x == items[i].x && g.y == items[i].y;
    }
    if (!same) return DASH_ERR_SCHEDULE_INVALID;
  }
  evict(g_tables);
  e.stamp = ++g_clock;
  *out = &g_tables.emplace(k, std::move(e)).first->second;
  return DASH_OK;
}

// A special mask's tables packed into pinned host memory as the
// workspace's table region from its unit offsets on (unit offsets | items |
// dead list), made on the first launch that needs them.  Caller holds g_mu.
dash_status pinned_blob(const MaskKey& key, TabEntry* e) {
  if (e->pinned) return DASH_OK;
  const MaskEntry* me = mask_entry(key);
  const Tables& t = e->host;
  const int n = key.n;
  const std::vector<int2> items = encode_items(t);
  const size_t items_at = align256(4 * (size_t)(n + 1));
  const size_t dead_at = align256(items_at + 8 * (size_t)std::max<long>(me->live_pairs, 1));
  const size_t bytes = dead_at + 4 * me->dead.size();
  char* p = nullptr;
  if (hipHostMalloc((void**)&p, bytes, hipHostMallocDefault) != hipSuccess) return DASH_ERR_HIP;
  std::memset(p, 0, bytes);
  std::memcpy(p, t.unit_off.data(), sizeof(int) * t.unit_off.size());
  if (!items.empty()) std::memcpy(p + items_at, items.data(), sizeof(int2) * items.size());
  if (!me->dead.empty()) std::memcpy(p + dead_at, me->dead.data(), 4 * me->dead.size());
  if (hipEventCreateWithFlags(&e->used, hipEventDisableTiming) != hipSuccess) {
    e->used = nullptr;
    (void)hipHostFree(p);
    return DASH_ERR_HIP;
  }
  e->pinned = p;
  e->bytes = bytes;
  return DASH_OK;
}

// Unit order of a dynamic ordered schedule: unit-major (unit 0 of every
// head, then unit 1, ...) when the DAG model predicts a makespan at least
// 5 % shorter than head by head for one group's share (the heads and
// workgroups of one XCD when units run in XCD groups).  A head's own units
// keep their relative order either way, so results are bit-identical; the
// order only changes which heads run side by side (masks whose units
// differ much in length gain most).  Caller holds g_mu.
bool unit_major_for(const MaskKey& mkey, const Tables& t, Sched s, long heads, int maxco,
                    bool grouped, const Cost& cost) {
  if (t.needs_static() || !t.ordered() || t.units() == 0) return false;
  const auto key = std::make_tuple(mkey, (int)s, heads, maxco, (int)grouped, cost);
  auto it = g_order.find(key);
  if (it != g_order.end()) return it->second;
  LaunchPrediction lp;
  const bool pick = launch_predict(t, heads, maxco, cost.data(), grouped, lp) && lp.unit_major;
  g_order[key] = pick;
  return pick;
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

// Whether some live pair hides elements (the kernel then masks them).
// Caller holds g_mu.
bool any_partial(const MaskKey& key) {
  if (plain_key(key)) return key.causal != 0;
  return mask_entry(key)->host.any_partial();
}

// The costs AUTO uses for (device, dtype, d): fitted by
// dash_attn_bwd_calibrate, else the defaults of the layout an automatic
// launch runs.  Caller holds g_mu.
Cost costs_for(int dev, int dtype, int d) {
  auto it = g_costs.find(std::make_tuple(dev, dtype, d));
  if (it != g_costs.end()) return it->second;
  const double* c = auto_layout(dtype, d) == kLayoutPipe ? kPipeCost : kDefaultCost;
  return Cost{c[0], c[1], c[2], c[3]};
}

AutoKey auto_key(int dev, const dash_attn_desc* d, const MaskKey& mkey, int maxco) {
  const int h = (int)std::min<long>((long)d->B * d->H, 1L << 30);
  return AutoKey(dev, (int)d->dtype, d->d, mkey, h, maxco);
}

// DASH_SCHED_AUTO -> the schedule dash_attn_bwd_tune measured fastest for
// this problem on this device, else the ordered schedule the model predicts
// fastest on `maxco` co-resident workgroups with the device's costs
// (cached); other schedules unchanged.  Caller holds g_mu.
dash_status resolve_schedule(dash_schedule schedule, int dev, const dash_attn_desc* desc,
                             const MaskKey& mkey, int maxco, Sched* s) {
  *s = (Sched)schedule;
  if (schedule != DASH_SCHED_AUTO) return DASH_OK;
  const AutoKey akey = auto_key(dev, desc, mkey, maxco);
  auto tt = g_tuned.find(akey);
  if (tt != g_tuned.end()) {
    *s = tt->second;
    return DASH_OK;
  }
  const Cost cost = costs_for(dev, desc->dtype, desc->d);
  const auto key = std::make_pair(akey, cost);
  auto it = g_auto.find(key);
  if (it != g_auto.end()) {
    *s = it->second;
    return DASH_OK;
  }
  double pred[3];
  if (plain_key(mkey) && mkey.n + 1 > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
  const dash::TileMask m = plain_key(mkey) ? dash::plain_mask(mkey.n, mkey.causal != 0)
                                           : mask_entry(mkey)->host;
  const dash_status st = choose_schedule(m, std::get<4>(akey), maxco, cost.data(), s, pred, true);
  if (st != DASH_OK) return st;
  g_auto[key] = *s;
  return DASH_OK;
}

// Reads the workspace's status word (synchronous copy; the caller has
// synchronized the stream the backward ran on).
dash_status read_status(const void* workspace) {
  if (workspace == DASH_NOALLOC_WORKSPACE) {
    void* p = nullptr;
    if (dash::noalloc_scratch(&p) != hipSuccess) return DASH_ERR_HIP;
    workspace = p;
  }
  uint32_t word = 0;
  if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return DASH_ERR_HIP;
  return word ? DASH_ERR_ORDER_TIMEOUT : DASH_OK;
}

// noalloc: the workspace is the built-in scratch; masks whose tables come
// from pinned host memory (allocated on first use) are refused.
dash_status run_bwd(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                    const void* k, const void* v, const void* dout, const float* lse,
                    const float* delta, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, const dash_bwd_debug* dbg, void* stream,
                    bool noalloc = false) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok_run(schedule)) return DASH_ERR_INVALID_ARG;
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv || !workspace)
    return DASH_ERR_INVALID_ARG;
  int bc = 0, br = 0;
  dash::bwd_tiles(desc->dtype, desc->d, &bc, &br);
  const int n = desc->N / bc;
  const bool ordered = schedule != DASH_SCHED_ATOMIC;
  if (dbg && (dbg->poison_q < 0 || dbg->poison_q > desc->N / br)) return DASH_ERR_INVALID_ARG;
  if (dbg && (dbg->placement < 0 || dbg->placement > 3)) return DASH_ERR_INVALID_ARG;
  if (dbg && (dbg->unit_order < 0 || dbg->unit_order > 2)) return DASH_ERR_INVALID_ARG;
  int lay = dbg ? dbg->layout : 0;
  if (lay < 0 || lay > kLayoutOneStage) return DASH_ERR_INVALID_ARG;
  const bool auto_lay = lay == 0;
  if (auto_lay) lay = auto_layout(desc->dtype, desc->d);
  if (lay == kLayoutPairs && (desc->dtype != DASH_BF16 || desc->d != 128)) return DASH_ERR_UNSUPPORTED;
  if (lay == kLayoutPipe && (desc->dtype != DASH_BF16 || (desc->d != 128 && desc->d != 64)))
    return DASH_ERR_UNSUPPORTED;

  const MaskKey mkey = mask_key(desc);
  const bool plain = plain_key(mkey);
  if (plain && n > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
  if (noalloc && !plain) return DASH_ERR_UNSUPPORTED;
  const long heads = (long)desc->B * desc->H;
  hipStream_t strm = (hipStream_t)stream;
  char* ws = (char*)workspace;

  std::unique_lock<std::mutex> lock(g_mu);
  const WsLayout w = layout(desc, live_pairs_of(mkey));
  if (workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return DASH_ERR_WORKSPACE;
  // elements are masked inside some pairs (causal diagonal, window edges)
  const bool masked = any_partial(mkey);
  lock.unlock();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  int maxco = 0;
  st = get_coresident(dev, desc->dtype, desc->d, masked, ordered, &maxco);
  if (st != DASH_OK) return st;
  if (lay != kLayoutOneStage) {
    // the 8-wave kernels must fit as many workgroups as the one-stage kernel
    // (the schedule's tables are planned for that many); an automatic launch
    // that finds fewer runs the one-stage kernel instead
    int pb = 0;
    if ((lay == kLayoutPairs ? dash::bwd_pair_max_coresident(masked, ordered, &pb)
                             : dash::bwd_pipe_max_coresident(desc->d, masked, ordered, &pb)) != hipSuccess)
      return DASH_ERR_HIP;
    if (pb < maxco) {
      if (!auto_lay) return DASH_ERR_UNSUPPORTED;
      lay = kLayoutOneStage;
    }
  }
  const bool pairs = lay == kLayoutPairs, pipe = lay == kLayoutPipe;
  lock.lock();
  Sched s = Sched::Naive;
  st = resolve_schedule(schedule, dev, desc, mkey, maxco, &s);
  if (st != DASH_OK) return st;
  TabEntry* tb = nullptr;
  st = tab_entry(mkey, s, plan_slots(mkey, s, heads, maxco), &tb);
  if (st != DASH_OK) return st;
  const Tables& host = tb->host;
  const int U = host.units();
  const long total_units = heads * U;
  int grid = 0, p_eff = 0, dynamic = 0;
  if (U == 0) {
    // no live pair at all: only the dead-tile clears below run
  } else if (host.needs_static()) {
    p_eff = (maxco / U) * U;
    if (p_eff < 1) return DASH_ERR_UNSUPPORTED;  // a whole head must be resident
    if (p_eff > total_units) p_eff = (int)total_units;
    grid = p_eff;
  } else {
    dynamic = 1;
    grid = (int)std::min<long>(maxco, total_units);
    p_eff = grid;
    // a timed shift needs enough workgroups to be deadlock-free device-wide
    // (the kernel checks its XCD groups itself)
    if (host.timed() && grid < dash::timed_need(host.slots_per_head, heads))
      return DASH_ERR_UNSUPPORTED;
  }
  int xcd_mode = ordered ? 1 : 0;
  if (dbg && dbg->placement) xcd_mode = dbg->placement - 1;
  int unit_major =
      dynamic ? (unit_major_for(mkey, host, s, heads, maxco, xcd_mode != 0,
                                costs_for(dev, desc->dtype, desc->d)) ? 1 : 0)
              : 0;
  if (dbg && dbg->unit_order && dynamic) unit_major = dbg->unit_order - 1;
  int n_dead_q = 0, n_dead_kv = 0;
  if (!plain) {
    const MaskEntry* me = mask_entry(mkey);
    n_dead_q = me->n_dead_q;
    n_dead_kv = me->n_dead_kv;
    st = pinned_blob(mkey, tb);
    if (st != DASH_OK) return st;
  }

  // workspace prologue: clear the header and counters (and, for the atomic
  // schedule, the accumulator); write a plain mask's tables.  Ordered
  // schedules never read an accumulator element before its first
  // contributor wrote it.
  dash::PrologueArgs pa;
  pa.clear = (uint32_t*)ws;
  pa.clear_words = w.unit_off_off / 4;
  pa.clear2 = ordered ? nullptr : (uint32_t*)(ws + w.acc_off);
  pa.clear2_words = ordered ? 0 : (w.total - w.acc_off) / 4;
  pa.n = plain ? n : 0;
  pa.causal = mkey.causal;
  pa.sched = (int)s;
  pa.units = U;
  pa.items = plain ? dash::plain::items(n, mkey.causal != 0) : 0;
  pa.unit_off = (int*)(ws + w.unit_off_off);
  pa.item = (int2*)(ws + w.items_off);
  // the pipeline layout reads LSE * log2(e), one product per row
  pa.lse = lse;
  pa.lse2 = (float*)(ws + w.lse2_off);
  pa.lse_count = pipe ? (size_t)heads * desc->N : 0;
  if (dash::launch_bwd_prologue(pa, strm) != hipSuccess) return DASH_ERR_HIP;
  if (!plain) {
    // special masks: the host-built tables, copied on the caller's stream
    if (hipMemcpyAsync(ws + w.unit_off_off, tb->pinned, tb->bytes, hipMemcpyHostToDevice, strm) !=
            hipSuccess ||
        hipEventRecord(tb->used, strm) != hipSuccess)
      return DASH_ERR_HIP;
  }
  lock.unlock();

  dash::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.lse2 = (const float*)(ws + w.lse2_off);
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_accum = (float*)(ws + w.acc_off);
  a.counters = (uint32_t*)(ws + w.counters_off);
  a.header = (uint32_t*)ws;
  a.unit_off = (const int*)(ws + w.unit_off_off);
  a.items = (const int2*)(ws + w.items_off);
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
  a.xcd_mode = xcd_mode;
  a.unit_major = unit_major;
  a.timed_slots = host.timed() ? host.slots_per_head : 0;
  a.scale = scale_of(desc);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.spin_limit = (dbg && dbg->spin_limit) ? dbg->spin_limit : kDefaultSpin;
  a.jitter_seed = dbg ? dbg->jitter_seed : 0u;
  a.poison_q = dbg ? dbg->poison_q - 1 : -1;
  a.partials = dbg ? dbg->partials : nullptr;
  a.wait_stats = dbg ? dbg->wait_stats : nullptr;
  a.phase_stats = dbg ? dbg->phase_stats : nullptr;
  // (the 8-wave layouts time 8 waves per workgroup)
  if ((a.wait_stats || a.phase_stats) &&
      (long)grid * ((pairs || pipe) ? 8 : dash::bwd_waves(desc->dtype, desc->d)) > 4096L * 4)
    return DASH_ERR_UNSUPPORTED;
  hipEvent_t ev0 = dbg ? (hipEvent_t)dbg->kernel_events[0] : nullptr;
  hipEvent_t ev1 = dbg ? (hipEvent_t)dbg->kernel_events[1] : nullptr;
  if (ev0 && hipEventRecord(ev0, strm) != hipSuccess) return DASH_ERR_HIP;
  if (U > 0 && (pairs  ? dash::launch_bwd_pair(masked, ordered, a, grid, strm)
                : pipe ? dash::launch_bwd_pipe(desc->d, masked, ordered, a, grid, strm)
                       : dash::launch_bwd(desc->dtype, desc->d, masked, ordered, a, grid, strm)) !=
                   hipSuccess)
    return DASH_ERR_HIP;
  if (ev1 && hipEventRecord(ev1, strm) != hipSuccess) return DASH_ERR_HIP;
  // gradient rows no pair touches: dQ of Q blocks that see no key (the
  // atomic path's conversion already writes them), dK and dV of KV tiles no
  // query sees
  const int* dead = (const int*)(ws + w.dead_off);
  if (ordered && n_dead_q &&
      dash::launch_zero_tiles(desc->dtype, dq, dead, n_dead_q, bc, desc->d, desc->N, (int)heads,
                              strm) != hipSuccess)
    return DASH_ERR_HIP;
  if (n_dead_kv) {
    if (dash::launch_zero_tiles(desc->dtype, dk, dead + n_dead_q, n_dead_kv, bc, desc->d, desc->N,
                                (int)heads, strm) != hipSuccess ||
        dash::launch_zero_tiles(desc->dtype, dv, dead + n_dead_q, n_dead_kv, bc, desc->d, desc->N,
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

// Runs NAIVE, DESCENDING and SHIFT (those that can run) once untimed and
// `reps` times timed on the caller's buffers, exactly as dash_attn_bwd
// would, and returns the mean time per launch (NaN where a schedule cannot
// run), reading the status word after each candidate (every launch clears
// it).  Blocking.  Reports the device and its co-resident workgroups.
dash_status time_schedules(const dash_attn_desc* desc, const void* q, const void* k,
                           const void* v, const void* dout, const float* lse, const float* delta,
                           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           int32_t reps, void* stream, float t[3], int* dev_out, int* maxco_out) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (reps < 1 || reps > 1000) return DASH_ERR_INVALID_ARG;
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv || !workspace)
    return DASH_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  const MaskKey mkey = mask_key(desc);
  bool masked = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    masked = any_partial(mkey);
  }
  int maxco = 0;
  st = get_coresident(dev, desc->dtype, desc->d, masked, true, &maxco);
  if (st != DASH_OK) return st;
  *dev_out = dev;
  *maxco_out = maxco;
  hipStream_t strm = (hipStream_t)stream;
  hipEvent_t ev[2];
  if (hipEventCreate(&ev[0]) != hipSuccess) return DASH_ERR_HIP;
  if (hipEventCreate(&ev[1]) != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return DASH_ERR_HIP;
  }
  const dash_schedule cand[3] = {DASH_SCHED_NAIVE, DASH_SCHED_DESCENDING, DASH_SCHED_SHIFT};
  const long bh = (long)desc->B * desc->H;
  for (int i = 0; i < 3 && st == DASH_OK; ++i) {
    t[i] = NAN;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      TabEntry* tb = nullptr;
      if (tab_entry(mkey, (Sched)cand[i], plan_slots(mkey, (Sched)cand[i], bh, maxco), &tb) !=
          DASH_OK)
        continue;
      if (tb->host.needs_static() && tb->host.units() > maxco) continue;
    }
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
    // every launch clears the status word, so a time-out of this
    // candidate is visible only now, before the next one runs
    st = read_status(workspace);
    if (st != DASH_OK) break;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) {
      st = DASH_ERR_HIP;
      break;
    }
    t[i] = ms / reps;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return st;
}

// Host entry points that build tables can run out of host memory; nothing
// may throw across the C boundary.
template <typename F>
dash_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return DASH_ERR_HOST_MEMORY;
  } catch (...) {
    return DASH_ERR_INVALID_ARG;
  }
}

// The DAG calculator numbers 2 nodes per item with 32-bit indices.
bool predict_fits(const Tables& t, long heads) {
  return 2.0 * (double)t.items() * (double)heads < 2147483647.0;
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
    case DASH_ERR_HOST_MEMORY: return "out of host memory";
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

size_t dash_attn_fwd_workspace_size(const dash_attn_desc* desc) {
  if (check_desc(desc) != DASH_OK) return 0;
  const MaskKey mkey = mask_key(desc);
  if (mkey.block.empty()) return 0;
  return align256((size_t)mkey.n * mkey.n);
}

dash_status dash_attn_fwd_ws(const dash_attn_desc* desc, const void* q, const void* k,
                             const void* v, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return guarded([&]() -> dash_status {
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
    hipStream_t strm = (hipStream_t)stream;
    std::unique_lock<std::mutex> lock(g_mu, std::defer_lock);
    if (!mkey.block.empty()) {
      // block masks: the tile liveness, copied into the caller's workspace
      const size_t bytes = (size_t)mkey.n * mkey.n;
      if (!workspace || workspace_bytes < align256(bytes) || ((uintptr_t)workspace & 255u))
        return DASH_ERR_WORKSPACE;
      lock.lock();
      MaskEntry* me = mask_entry(mkey);
      if (!me->pinned_live) {
        if (hipHostMalloc((void**)&me->pinned_live, bytes, hipHostMallocDefault) != hipSuccess) {
          me->pinned_live = nullptr;
          return DASH_ERR_HIP;
        }
        std::memcpy(me->pinned_live, me->host.live.data(), bytes);
      }
      if (!me->used && hipEventCreateWithFlags(&me->used, hipEventDisableTiming) != hipSuccess) {
        me->used = nullptr;
        return DASH_ERR_HIP;
      }
      if (hipMemcpyAsync(workspace, me->pinned_live, bytes, hipMemcpyHostToDevice, strm) !=
              hipSuccess ||
          hipEventRecord(me->used, strm) != hipSuccess)
        return DASH_ERR_HIP;
      lock.unlock();
      a.live = (const uint8_t*)workspace;
    }
    if (dash::launch_fwd(desc->dtype, desc->d, mkey.masked(), a, strm) != hipSuccess)
      return DASH_ERR_HIP;
    return DASH_OK;
  });
}

dash_status dash_attn_fwd(const dash_attn_desc* desc, const void* q, const void* k, const void* v,
                          void* o, float* lse, void* stream) {
  return dash_attn_fwd_ws(desc, q, k, v, o, lse, nullptr, 0, stream);
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

size_t dash_attn_bwd_workspace_size(const dash_attn_desc* desc, dash_schedule schedule) {
  if (check_desc(desc) != DASH_OK || !sched_ok_run(schedule)) return 0;
  try {
    const MaskKey mkey = mask_key(desc);
    // longer units than the kernel stages cannot run
    if (plain_key(mkey) && mkey.n > dash::kMaxUnitItems) return 0;
    std::lock_guard<std::mutex> lock(g_mu);
    return layout(desc, live_pairs_of(mkey)).total;
  } catch (...) {
    return 0;
  }
}

dash_status dash_attn_bwd(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                          const void* k, const void* v, const void* dout, const float* lse,
                          const float* delta, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return guarded([&] {
    return run_bwd(desc, schedule, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                   workspace_bytes, nullptr, stream);
  });
}

dash_status dash_attn_bwd_noalloc(const dash_attn_desc* desc, dash_schedule schedule,
                                  const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, const float* delta, void* dq, void* dk,
                                  void* dv, void* stream) {
  return guarded([&]() -> dash_status {
    dash_status st = check_desc(desc);
    if (st != DASH_OK) return st;
    if (!sched_ok_run(schedule)) return DASH_ERR_INVALID_ARG;
    size_t need = 0;
    {
      const MaskKey mkey = mask_key(desc);
      if (!plain_key(mkey)) return DASH_ERR_UNSUPPORTED;
      if (mkey.n > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
      std::lock_guard<std::mutex> lock(g_mu);
      need = layout(desc, live_pairs_of(mkey)).total;
    }
    if (need > dash::kNoallocScratchBytes) return DASH_ERR_WORKSPACE;
    void* ws = nullptr;
    if (dash::noalloc_scratch(&ws) != hipSuccess) return DASH_ERR_HIP;
    return run_bwd(desc, schedule, q, k, v, dout, lse, delta, dq, dk, dv, ws,
                   dash::kNoallocScratchBytes, nullptr, stream, true);
  });
}

dash_status dash_attn_bwd_debug(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                                const void* k, const void* v, const void* dout, const float* lse,
                                const float* delta, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, const dash_bwd_debug* dbg, void* stream) {
  if (!dbg) return DASH_ERR_INVALID_ARG;
  return guarded([&] {
    return run_bwd(desc, schedule, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                   workspace_bytes, dbg, stream);
  });
}

dash_status dash_attn_bwd_tune(const dash_attn_desc* desc, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, int32_t reps, dash_schedule* choice,
                              float* times_ms, void* stream) {
  return guarded([&]() -> dash_status {
    if (!choice) return DASH_ERR_INVALID_ARG;
    float t[3];
    int dev = 0, maxco = 0;
    const dash_status st = time_schedules(desc, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                                          workspace_bytes, reps, stream, t, &dev, &maxco);
    if (st != DASH_OK) return st;
    const dash_schedule cand[3] = {DASH_SCHED_NAIVE, DASH_SCHED_DESCENDING, DASH_SCHED_SHIFT};
    int best = -1;
    for (int i = 0; i < 3; ++i)
      if (std::isfinite(t[i]) && (best < 0 || t[i] < t[best])) best = i;
    if (best < 0) return DASH_ERR_UNSUPPORTED;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      g_tuned[auto_key(dev, desc, mask_key(desc), maxco)] = (Sched)cand[best];
    }
    *choice = cand[best];
    if (times_ms) std::memcpy(times_ms, t, sizeof(t));
    return DASH_OK;
  });
}

dash_status dash_attn_bwd_calibrate(const dash_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const void* dout, const float* lse,
                                    const float* delta, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes, int32_t reps,
                                    double cost_out[4], double* residual, float* times_ms,
                                    void* stream) {
  return guarded([&]() -> dash_status {
    float t[3];
    int dev = 0, maxco = 0;
    dash_status st = time_schedules(desc, q, k, v, dout, lse, delta, dq, dk, dv, workspace,
                                    workspace_bytes, reps, stream, t, &dev, &maxco);
    if (st != DASH_OK) return st;
    if (times_ms) std::memcpy(times_ms, t, sizeof(t));
    const double ms[3] = {t[0], t[1], t[2]};
    const MaskKey mkey = mask_key(desc);
    Cost c;
    double res = 0.0;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      const dash::TileMask m = plain_key(mkey) ? dash::plain_mask(mkey.n, mkey.causal != 0)
                                               : mask_entry(mkey)->host;
      st = fit_costs(m, (long)desc->B * desc->H, maxco, ms, c, &res, nullptr);
      if (st != DASH_OK) return st;
      g_costs[std::make_tuple(dev, (int)desc->dtype, desc->d)] = c;
    }
    if (cost_out) std::memcpy(cost_out, c.data(), sizeof(double) * 4);
    if (residual) *residual = res;
    return DASH_OK;
  });
}

dash_status dash_attn_bwd_costs(const dash_attn_desc* desc, double cost_out[4]) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!cost_out) return DASH_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  const Cost c = costs_for(dev, desc->dtype, desc->d);
  std::memcpy(cost_out, c.data(), sizeof(double) * 4);
  return DASH_OK;
}

dash_status dash_schedule_fit_costs(const dash_attn_desc* desc, int32_t slots,
                                    const double ms[3], double cost_out[4], double* residual,
                                    double* item_ms) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (slots < 1 || !ms || !cost_out) return DASH_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (ms[i] < 0.0) return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    const MaskKey mkey = mask_key(desc);
    if (plain_key(mkey) && mkey.n + 1 > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    const dash::TileMask m = plain_key(mkey) ? dash::plain_mask(mkey.n, mkey.causal != 0)
                                             : mask_entry(mkey)->host;
    Cost c;
    const dash_status st2 = fit_costs(m, (long)desc->B * desc->H, slots, ms, c, residual, item_ms);
    if (st2 != DASH_OK) return st2;
    std::memcpy(cost_out, c.data(), sizeof(double) * 4);
    return DASH_OK;
  });
}

dash_status dash_status_query(const void* workspace) {
  if (!workspace) return DASH_ERR_INVALID_ARG;
  return read_status(workspace);
}

dash_status dash_attn_bwd_status(const void* workspace, void* stream) {
  if (!workspace) return DASH_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DASH_ERR_HIP;
  return read_status(workspace);
}

dash_status dash_schedule_tables(int32_t n, int32_t causal, dash_schedule schedule,
                                 int32_t* n_units, int32_t* unit_offsets, int32_t* item_kv,
                                 int32_t* item_q, int32_t* rank) {
  if (n < 1 || n > 32767 || (causal != 0 && causal != 1) || !sched_ok(schedule) || !n_units ||
      !unit_offsets || !item_kv || !item_q || !rank)
    return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    Tables t;
    if (!dash::build_tables(n, causal != 0, (Sched)schedule, t)) return DASH_ERR_UNSUPPORTED;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    *n_units = t.units();
    std::memcpy(unit_offsets, t.unit_off.data(), sizeof(int) * t.unit_off.size());
    std::memcpy(item_kv, t.kv.data(), sizeof(int) * t.kv.size());
    std::memcpy(item_q, t.q.data(), sizeof(int) * t.q.size());
    std::memcpy(rank, t.rank.data(), sizeof(int) * t.rank.size());
    return DASH_OK;
  });
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
  return guarded([&]() -> dash_status {
    const MaskKey mkey = mask_key(desc);
    if (plain_key(mkey) && mkey.n + 1 > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
    int ws = 0;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      ws = plan_slots(mkey, (Sched)schedule, (long)desc->B * desc->H, slots);
    }
    Tables t;
    if (!dash::build_tables(tile_mask(mkey), (Sched)schedule, t, ws > 0 ? ws : 1))
      return DASH_ERR_UNSUPPORTED;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    if (t.needs_static() && t.units() > slots) return DASH_ERR_UNSUPPORTED;
    const long heads = (long)desc->B * desc->H;
    if (!predict_fits(t, heads)) return DASH_ERR_UNSUPPORTED;
    dash::DagResult r;
    if (!dash::dag_predict(t, (int)heads, slots, cost, r, unit_major != 0))
      return DASH_ERR_SCHEDULE_INVALID;
    out[0] = r.makespan;
    out[1] = r.total_wait;
    out[2] = r.max_slot_idle;
    out[3] = r.lower_bound;
    return DASH_OK;
  });
}

dash_status dash_attn_bwd_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                  int32_t slots, const double cost[4], double out[4],
                                  int32_t info[4]) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok(schedule) || slots < 1 || !cost || !out) return DASH_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!(cost[i] >= 0.0) || !std::isfinite(cost[i])) return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    const MaskKey mkey = mask_key(desc);
    if (plain_key(mkey) && mkey.n + 1 > dash::kMaxUnitItems) return DASH_ERR_UNSUPPORTED;
    int ws = 0;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      ws = plan_slots(mkey, (Sched)schedule, (long)desc->B * desc->H, slots);
    }
    Tables t;
    if (!dash::build_tables(tile_mask(mkey), (Sched)schedule, t, ws > 0 ? ws : 1))
      return DASH_ERR_UNSUPPORTED;
    if (dash::validate_tables(t)[0] != '\0') return DASH_ERR_SCHEDULE_INVALID;
    if (t.needs_static() && t.units() > slots) return DASH_ERR_UNSUPPORTED;
    LaunchPrediction lp;
    if (!launch_predict(t, (long)desc->B * desc->H, slots, cost, schedule != DASH_SCHED_ATOMIC,
                        lp))
      return DASH_ERR_SCHEDULE_INVALID;
    out[0] = lp.r.makespan;
    out[1] = lp.r.total_wait;
    out[2] = lp.r.max_slot_idle;
    out[3] = lp.r.lower_bound;
    if (info) {
      info[0] = lp.groups;
      info[1] = lp.unit_major;
      info[2] = lp.heads;
      info[3] = lp.slots;
    }
    return DASH_OK;
  });
}

dash_status dash_schedule_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                  int32_t slots, const double cost[4], double out[4]) {
  return dash_attn_schedule_predict(desc, schedule, slots, 0, cost, out);
}

dash_status dash_attn_bwd_resolve_schedule(const dash_attn_desc* desc, dash_schedule schedule,
                                           dash_schedule* resolved) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok_run(schedule) || !resolved) return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
    const MaskKey mkey = mask_key(desc);
    bool masked = false;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      masked = any_partial(mkey);
    }
    int maxco = 0;
    dash_status st2 = get_coresident(dev, desc->dtype, desc->d, masked,
                                     schedule != DASH_SCHED_ATOMIC, &maxco);
    if (st2 != DASH_OK) return st2;
    Sched s = Sched::Naive;
    std::lock_guard<std::mutex> lock(g_mu);
    st2 = resolve_schedule(schedule, dev, desc, mkey, maxco, &s);
    if (st2 != DASH_OK) return st2;
    *resolved = (dash_schedule)s;
    return DASH_OK;
  });
}

dash_status dash_schedule_choose(int32_t n, int32_t causal, int32_t heads, int32_t slots,
                                 const double* cost, dash_schedule* choice, double* predicted) {
  if (n < 1 || n > 32767 || (causal != 0 && causal != 1) || heads < 1 || slots < 1 || !choice)
    return DASH_ERR_INVALID_ARG;
  const double* c = cost ? cost : kDefaultCost;
  for (int i = 0; i < 4; ++i)
    if (!(c[i] >= 0.0) || !std::isfinite(c[i])) return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    Sched s = Sched::Naive;
    double pred[3];
    const dash_status st =
        choose_schedule(dash::plain_mask(n, causal != 0), heads, slots, c, &s, pred);
    if (st != DASH_OK) return st;
    *choice = (dash_schedule)s;
    if (predicted) std::memcpy(predicted, pred, sizeof(pred));
    return DASH_OK;
  });
}

dash_status dash_attn_schedule_tables(const dash_attn_desc* desc, dash_schedule schedule,
                                      int32_t slots, int32_t sizes[5], int32_t* unit_offsets,
                                      int32_t* item_kv, int32_t* item_q, int32_t* item_step,
                                      uint8_t* item_partial, int32_t* rank) {
  dash_status st = check_desc(desc);
  if (st != DASH_OK) return st;
  if (!sched_ok(schedule) || !sizes || slots < 0) return DASH_ERR_INVALID_ARG;
  return guarded([&]() -> dash_status {
    const MaskKey mkey = mask_key(desc);
    int maxco = slots;
    if (maxco == 0) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
      bool masked = false;
      {
        std::lock_guard<std::mutex> lock(g_mu);
        masked = any_partial(mkey);
      }
      const dash_status st2 = get_coresident(dev, desc->dtype, desc->d, masked,
                                             schedule != DASH_SCHED_ATOMIC, &maxco);
      if (st2 != DASH_OK) return st2;
    }
    Tables t;
    {
      // the tables a launch runs: for a plain mask this also checks them
      // against the closed forms the device writes
      std::lock_guard<std::mutex> lock(g_mu);
      TabEntry* tb = nullptr;
      const int ws = plan_slots(mkey, (Sched)schedule, (long)desc->B * desc->H, maxco);
      const dash_status st2 = tab_entry(mkey, (Sched)schedule, ws, &tb);
      if (st2 != DASH_OK) return st2;
      t = tb->host;
    }
    const bool fill = unit_offsets && item_kv && item_q && item_step && item_partial && rank;
    if (fill && (sizes[0] != t.n || sizes[1] != t.units() || sizes[2] != t.items()))
      return DASH_ERR_INVALID_ARG;
    sizes[0] = t.n;
    sizes[1] = t.units();
    sizes[2] = t.items();
    sizes[3] = t.needs_static() ? 1 : 0;
    sizes[4] = t.slots_per_head;
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
  });
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
  return guarded([&]() -> dash_status {
    if (!dash::dag_longest_path(n_nodes, weights, n_edges, src, dst, latency, start, finish))
      return DASH_ERR_SCHEDULE_INVALID;
    return DASH_OK;
  });
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
