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
#include "schedule.hpp"

#include <algorithm>
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
      if (!t.causal || kv <= q) t.rank[(size_t)q * n + kv] = r++;
  }
}

void ranks_by_step(Tables& t) {
  const int n = t.n;
  // (step, unit, kv) per Q block, sorted
  std::vector<std::vector<std::array<int, 3>>> per_q(n);
  for (int u = 0; u < t.units(); ++u)
    for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i)
      per_q[t.q[i]].push_back({i - t.unit_off[u], u, t.kv[i]});
  for (int q = 0; q < n; ++q) {
    std::sort(per_q[q].begin(), per_q[q].end());
    for (size_t r = 0; r < per_q[q].size(); ++r) t.rank[(size_t)q * n + per_q[q][r][2]] = (int)r;
  }
}

}  // namespace

bool build_tables(int n, bool causal, Sched s, Tables& t) {
  t = Tables();
  t.n = n;
  t.causal = causal;
  t.sched = s;
  if (n < 1) return false;
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
  if (s == Sched::Naive || s == Sched::Descending) ranks_by_kv(t);
  else if (s == Sched::Shift) ranks_by_step(t);
  return true;
}

const char* validate_tables(const Tables& t) {
  const int n = t.n;
  if (n < 1 || t.unit_off.empty() || t.unit_off.front() != 0 || t.unit_off.back() != t.items())
    return "malformed unit offsets";
  std::vector<int> seen((size_t)n * n, 0), unit_of((size_t)n * n, -1), pos((size_t)n * n, -1);
  for (int u = 0; u < t.units(); ++u) {
    if (t.unit_off[u] > t.unit_off[u + 1]) return "malformed unit offsets";
    int last_kv = -1;
    std::vector<int> done_kv;
    for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i) {
      const int kv = t.kv[i], q = t.q[i];
      if (kv < 0 || kv >= n || q < 0 || q >= n) return "tile index out of range";
      if (t.causal && kv > q) return "masked pair scheduled";
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
      if ((!t.causal || kv <= q) && seen[(size_t)q * n + kv] != 1) return "live pair missing";
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
  if (!t.ordered()) return "";
  // rank rows are permutations
  std::vector<int> pred_item((size_t)t.items(), -1);
  for (int q = 0; q < n; ++q) {
    std::vector<int> by_rank(n, -1);
    int cnt = 0;
    for (int kv = 0; kv < n; ++kv) {
      const int r = t.rank[(size_t)q * n + kv];
      const bool live = !t.causal || kv <= q;
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
      if (!t.needs_static() && unit_of[(size_t)q * n + by_rank[r - 1]] >= unit_of[(size_t)q * n + by_rank[r]])
        return "wait on a later unit under the dynamic policy";
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
