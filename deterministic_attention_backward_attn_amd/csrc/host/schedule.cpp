// Schedule layer (DASH explainer, "Technisches Resuemee" 2.2 A and B; the
// authors' abstract, strategies (i) and (ii)).
//
//   Naive       one unit per KV tile, Q blocks ascending; dQ order = KV
//               tiles ascending (the fixed baseline order).
//   Descending  same units and dQ order, Q blocks visited last to first.
//   Shift/full  unit i visits Q blocks i, i+1, ..., n-1, 0, ..., i-1; a
//               block's dQ order is the step at which units reach it, so
//               concurrent units never meet on a block.
//   Shift/causal (symmetric shift) unit w pairs KV tiles w and n-1-w (n+1
//               items), phase 1 the dense square (Q blocks n/2..n-1 x KV
//               tiles 0..n/2-1) with a cyclic offset, phase 2 the two folded
//               triangles with a cyclic offset over n/2+1 super-rows; dQ
//               order by step.
//   Atomic      Naive's traversal, no order.
//
// Masks other than full and causal (windows, block masks) keep the same
// Naive / Descending / Atomic rules over the live pairs; Shift becomes a
// timed shift (see build_tables in schedule.hpp).
#include "schedule.hpp"

#include <algorithm>
#include <queue>
#include <array>
#include <tuple>

namespace dash {

namespace {

struct Builder {
  Tables& t;
  explicit Builder(Tables& tt) : t(tt) {}
  void open() { t.unit_off.push_back((int)t.kv.size()); }
  void add(int kv, int q) {
    t.kv.push_back(kv);
    t.q.push_back(q);
  }
  void finish() { t.unit_off.push_back((int)t.kv.size()); }
};

void ranks_by_kv(Tables& t) {
  const int n = t.n;
  for (int q = 0; q < n; ++q) {
    int r = 0;
    for (int kv = 0; kv < n; ++kv)
      if (t.live[(size_t)q * n + kv]) t.rank[(size_t)q * n + kv] = r++;
  }
}

void ranks_by_step(Tables& t) {
  const int n = t.n;
  // (step, unit, kv) per Q block, sorted
  std::vector<std::vector<std::array<int, 3>>> per_q(n);
  for (int u = 0; u < t.units(); ++u)
    for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i)
      per_q[t.q[i]].push_back({t.step[i], u, t.kv[i]});
  for (int q = 0; q < n; ++q) {
    std::sort(per_q[q].begin(), per_q[q].end());
    for (size_t r = 0; r < per_q[q].size(); ++r) t.rank[(size_t)q * n + per_q[q][r][2]] = (int)r;
  }
}

// Timed shift (declared with build_tables): a step-by-step simulation of
// `slots` workgroups running the units of one head.
void timed_shift(const TileMask& m, int slots, Tables& t) {
  const int n = m.n;
  std::vector<int> len(n, 0), order;
  for (int kv = 0; kv < n; ++kv) {
    for (int q = 0; q < n; ++q) len[kv] += m.live[(size_t)q * n + kv] ? 1 : 0;
    if (len[kv]) order.push_back(kv);
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return len[a] > len[b]; });
  const int U = (int)order.size();
  // each unit's Q blocks in cyclic order from its diagonal; a unit takes
  // the first one not yet used by itself and not taken by another unit at
  // this step (scanned from `head`, the first one it has not used)
  std::vector<std::vector<int>> cyc(n);
  std::vector<std::vector<uint8_t>> used(n);
  std::vector<int> head(n, 0);
  for (int kv : order) {
    for (int d = 0; d < n; ++d) {
      const int q = (kv + d) % n;
      if (m.live[(size_t)q * n + kv]) cyc[kv].push_back(q);
    }
    used[kv].assign(cyc[kv].size(), 0);
  }
  std::vector<std::vector<std::pair<int, int>>> got(n);  // per KV tile: (step, q)
  std::vector<int> taken(n, -1);                         // step at which q was last taken
  std::vector<int> running, start(n, -1);
  int next = 0;
  for (int step = 0; next < U || !running.empty(); ++step) {
    while ((int)running.size() < slots && next < U) {
      start[order[next]] = step;
      running.push_back(order[next++]);
    }
    for (int kv : running) {
      const std::vector<int>& c = cyc[kv];
      int& h = head[kv];
      while (h < (int)c.size() && used[kv][h]) ++h;
      for (int i = h; i < (int)c.size(); ++i) {
        if (used[kv][i] || taken[c[i]] == step) continue;
        used[kv][i] = 1;
        taken[c[i]] = step;
        got[kv].push_back(std::make_pair(step, c[i]));
        break;
      }
    }
    running.erase(std::remove_if(running.begin(), running.end(),
                                 [&](int kv) { return got[kv].size() == cyc[kv].size(); }),
                  running.end());
  }
  for (int kv : order) {
    t.unit_off.push_back((int)t.kv.size());
    t.unit_start.push_back(start[kv]);
    for (const auto& e : got[kv]) {
      t.kv.push_back(kv);
      t.q.push_back(e.second);
      t.step.push_back(e.first);
    }
  }
  t.slots_per_head = U > 0 ? std::min(slots, U) : 0;  // no unit: nothing to time
}

}  // namespace

bool TileMask::any_partial() const {
  for (uint8_t p : partial)
    if (p) return true;
  return false;
}

TileMask plain_mask(int n, bool causal) {
  TileMask m;
  m.n = n;
  m.causal = causal;
  m.plain = true;
  m.live.assign((size_t)n * n, 0);
  m.partial.assign((size_t)n * n, 0);
  for (int q = 0; q < n; ++q)
    for (int kv = 0; kv < n; ++kv) {
      m.live[(size_t)q * n + kv] = (!causal || kv <= q) ? 1 : 0;
      m.partial[(size_t)q * n + kv] = (causal && kv == q) ? 1 : 0;
    }
  return m;
}

void mask_bounds(bool causal, int window, int* lo, int* hi) {
  constexpr int kUnbounded = 1 << 30;
  *lo = causal ? 0 : -kUnbounded;
  *hi = kUnbounded;
  if (window > 0) {
    *hi = window - 1;
    if (!causal) *lo = -(window - 1);
  }
}

TileMask make_mask(int n, int tile, bool causal, int window, const uint8_t* block, int bt) {
  if (!block && (window <= 0 || (long long)window >= (long long)n * tile))
    return plain_mask(n, causal);
  int lo = 0, hi = 0;
  mask_bounds(causal, window, &lo, &hi);
  TileMask m;
  m.n = n;
  m.causal = causal;
  m.plain = false;
  m.live.assign((size_t)n * n, 0);
  m.partial.assign((size_t)n * n, 0);
  const int nb = block ? n / bt : 0;
  for (int q = 0; q < n; ++q)
    for (int kv = 0; kv < n; ++kv) {
      // i - j over the pair spans [(q-kv)T - (T-1), (q-kv)T + (T-1)]
      const long long a = (long long)(q - kv) * tile - (tile - 1);
      const long long b = (long long)(q - kv) * tile + (tile - 1);
      const bool any = a <= hi && b >= lo;
      const bool all = a >= lo && b <= hi;
      const bool blk = !block || block[(size_t)(q / bt) * nb + kv / bt] != 0;
      m.live[(size_t)q * n + kv] = (any && blk) ? 1 : 0;
      m.partial[(size_t)q * n + kv] = (any && blk && !all) ? 1 : 0;
    }
  return m;
}

bool build_tables(const TileMask& m, Sched s, Tables& t, int slots) {
  if (m.plain) return build_tables(m.n, m.causal, s, t);
  t = Tables();
  const int n = m.n;
  t.n = n;
  t.causal = m.causal;
  t.sched = s;
  t.static_policy = false;
  if (n < 1 || slots < 1) return false;
  t.live = m.live;
  t.partial = m.partial;
  t.rank.assign((size_t)n * n, -1);
  Builder b(t);
  if (s == Sched::Shift) {
    timed_shift(m, slots, t);
  } else {
    for (int kv = 0; kv < n; ++kv) {
      bool opened = false;
      for (int k = 0; k < n; ++k) {
        const int q = (s == Sched::Descending) ? n - 1 - k : k;
        if (!m.live[(size_t)q * n + kv]) continue;
        if (!opened) b.open();
        opened = true;
        b.add(kv, q);
      }
    }
  }
  b.finish();
  if (s == Sched::Naive || s == Sched::Descending) ranks_by_kv(t);
  else if (s == Sched::Shift) ranks_by_step(t);
  return true;
}

int timed_slots(int maxco, long heads, int units) {
  if (maxco < 1 || heads < 1 || units < 1) return 1;
  const long grid = std::min<long>(maxco, heads * units);
  long ws = (grid - 1) / heads + 1;  // device-wide
  const int g = maxco / 8;
  if (g >= 1) ws = std::min<long>(ws, (g - 1) / ((heads + 7) / 8) + 1);  // XCD groups
  return (int)std::max<long>(1, std::min<long>(ws, units));
}

bool build_tables(int n, bool causal, Sched s, Tables& t) {
  t = Tables();
  t.n = n;
  t.causal = causal;
  t.sched = s;
  t.static_policy = s == Sched::Shift;
  if (n < 1) return false;
  {
    TileMask pm = plain_mask(n, causal);
    t.live = std::move(pm.live);
    t.partial = std::move(pm.partial);
  }
  t.rank.assign((size_t)n * n, -1);
  Builder b(t);
  switch (s) {
    case Sched::Atomic:
    case Sched::Naive:
      for (int kv = 0; kv < n; ++kv) {
        b.open();
        for (int q = causal ? kv : 0; q < n; ++q) b.add(kv, q);
      }
      break;
    case Sched::Descending:
      for (int kv = 0; kv < n; ++kv) {
        b.open();
        const int lo = causal ? kv : 0;
        for (int q = n - 1; q >= lo; --q) b.add(kv, q);
      }
      break;
    case Sched::Shift:
      if (!causal) {
        for (int i = 0; i < n; ++i) {
          b.open();
          for (int step = 0; step < n; ++step) b.add(i, (i + step) % n);
        }
      } else if (n == 1) {
        b.open();
        b.add(0, 0);
      } else {
        if (n % 2) return false;
        const int h = n / 2;
        for (int w = 0; w < h; ++w) {
          b.open();
          for (int step = 0; step < h; ++step) b.add(w, h + (w + step) % h);  // dense square
          for (int step = 0; step <= h; ++step) {                              // folded part
            const int k = (w + step) % (h + 1);
            if (k == h) b.add(n - 1 - w, n - 1);
            else if (k == h - 1 || w <= k) b.add(w, k);
            else b.add(n - 1 - w, n - 2 - k);
          }
        }
      }
      break;
  }
  // close: unit_off holds each unit's start; append the end
  b.finish();
  if (s == Sched::Shift) {
    t.step.assign(t.kv.size(), 0);
    for (int u = 0; u < t.units(); ++u)
      for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i) t.step[i] = i - t.unit_off[u];
  }
  if (s == Sched::Naive || s == Sched::Descending) ranks_by_kv(t);
  else if (s == Sched::Shift) ranks_by_step(t);
  return true;
}

const char* validate_tables(const Tables& t) {
  const int n = t.n;
  if (n < 1 || t.unit_off.empty() || t.unit_off.front() != 0 || t.unit_off.back() != t.items())
    return "malformed unit offsets";
  if (t.live.size() != (size_t)n * n || t.partial.size() != (size_t)n * n)
    return "malformed liveness";
  std::vector<int> seen((size_t)n * n, 0), unit_of((size_t)n * n, -1), pos((size_t)n * n, -1);
  for (int u = 0; u < t.units(); ++u) {
    if (t.unit_off[u] > t.unit_off[u + 1]) return "malformed unit offsets";
    int last_kv = -1;
    std::vector<int> done_kv;
    for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i) {
      const int kv = t.kv[i], q = t.q[i];
      if (kv < 0 || kv >= n || q < 0 || q >= n) return "tile index out of range";
      if (!t.live[(size_t)q * n + kv]) return "dead pair scheduled";
      if (seen[(size_t)q * n + kv]++) return "pair scheduled twice";
      unit_of[(size_t)q * n + kv] = u;
      pos[(size_t)q * n + kv] = i;
      if (kv != last_kv) {
        if (std::find(done_kv.begin(), done_kv.end(), kv) != done_kv.end())
          return "KV tile split within a unit";
        if (last_kv >= 0) done_kv.push_back(last_kv);
        last_kv = kv;
      }
    }
  }
  for (int q = 0; q < n; ++q)
    for (int kv = 0; kv < n; ++kv)
      if (t.live[(size_t)q * n + kv] && seen[(size_t)q * n + kv] != 1) return "live pair missing";
  // KV tile must live in one unit only
  for (int kv = 0; kv < n; ++kv) {
    int u0 = -1;
    for (int q = 0; q < n; ++q) {
      const int u = unit_of[(size_t)q * n + kv];
      if (u < 0) continue;
      if (u0 < 0) u0 = u;
      else if (u != u0) return "KV tile spread over units";
    }
  }
  if (!t.step.empty()) {
    // lockstep steps: increasing within a unit, distinct within a Q block
    if (t.step.size() != t.kv.size()) return "malformed steps";
    for (int u = 0; u < t.units(); ++u)
      for (int i = t.unit_off[u] + 1; i < t.unit_off[u + 1]; ++i)
        if (t.step[i] <= t.step[i - 1]) return "steps not increasing within a unit";
    std::vector<std::vector<int>> per_q(n);
    for (int i = 0; i < t.items(); ++i) per_q[t.q[i]].push_back(t.step[i]);
    for (auto& v : per_q) {
      std::sort(v.begin(), v.end());
      if (std::adjacent_find(v.begin(), v.end()) != v.end()) return "two units on one block at one step";
    }
  }
  if (t.timed()) {
    // the timing certificate: units listed in start order, and at most
    // slots_per_head units between their first and last step at any step
    if (t.step.empty() || t.needs_static() || (int)t.unit_start.size() != t.units())
      return "malformed timed tables";
    std::vector<int> opens, closes;
    for (int u = 0; u < t.units(); ++u) {
      if (t.unit_off[u] == t.unit_off[u + 1]) return "empty unit";
      opens.push_back(t.unit_start[u]);
      closes.push_back(t.step[t.unit_off[u + 1] - 1]);
      if (opens[u] < 0 || t.step[t.unit_off[u]] < opens[u]) return "item before its unit's start";
      if (u > 0 && opens[u] < opens[u - 1]) return "units not in start order";
    }
    std::sort(closes.begin(), closes.end());
    // units running at the step where unit u starts: started at or before
    // it (listed no later) and not closed before it
    for (int u = 0; u < t.units(); ++u) {
      const long closed_before =
          std::lower_bound(closes.begin(), closes.end(), opens[u]) - closes.begin();
      const long started = std::upper_bound(opens.begin(), opens.end(), opens[u]) - opens.begin();
      if (started - closed_before > t.slots_per_head) return "more units running than slots";
    }
  }
  if (!t.ordered()) return "";
  // rank rows are permutations
  std::vector<int> pred_item((size_t)t.items(), -1);
  for (int q = 0; q < n; ++q) {
    std::vector<int> by_rank(n, -1);
    int cnt = 0;
    for (int kv = 0; kv < n; ++kv) {
      const int r = t.rank[(size_t)q * n + kv];
      const bool live = t.live[(size_t)q * n + kv] != 0;
      if (!live) {
        if (r != -1) return "rank for a masked pair";
        continue;
      }
      if (r < 0 || r >= n || by_rank[r] != -1) return "rank row is not a permutation";
      by_rank[r] = kv;
      ++cnt;
    }
    for (int r = 0; r < cnt; ++r)
      if (by_rank[r] < 0) return "rank row is not a permutation";
    for (int r = 1; r < cnt; ++r) {
      const int cur = pos[(size_t)q * n + by_rank[r]];
      const int prev = pos[(size_t)q * n + by_rank[r - 1]];
      pred_item[cur] = prev;
      if (t.timed()) {
        if (t.step[prev] >= t.step[cur]) return "dQ order is not by step";
      } else if (!t.needs_static() &&
                 unit_of[(size_t)q * n + by_rank[r - 1]] >= unit_of[(size_t)q * n + by_rank[r]]) {
        return "wait on a later unit under the dynamic policy";
      }
    }
  }
  // item-level graph of one head (unit chains + order edges) must be acyclic
  const int m = t.items();
  std::vector<int> indeg(m, 0);
  std::vector<std::vector<int>> succ(m);
  for (int u = 0; u < t.units(); ++u)
    for (int i = t.unit_off[u] + 1; i < t.unit_off[u + 1]; ++i) {
      succ[i - 1].push_back(i);
      ++indeg[i];
    }
  for (int i = 0; i < m; ++i)
    if (pred_item[i] >= 0) {
      succ[pred_item[i]].push_back(i);
      ++indeg[i];
    }
  std::vector<int> stack;
  for (int i = 0; i < m; ++i)
    if (!indeg[i]) stack.push_back(i);
  int visited = 0;
  while (!stack.empty()) {
    const int x = stack.back();
    stack.pop_back();
    ++visited;
    for (int y : succ[x])
      if (--indeg[y] == 0) stack.push_back(y);
  }
  if (visited != m) return "dependency cycle";
  return "";
}

}  // namespace dash
