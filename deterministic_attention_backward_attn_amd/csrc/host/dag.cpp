// DAG critical-path calculator: see dag.hpp for the model.
#include "dag.hpp"

#include <algorithm>
#include <functional>
#include <queue>
#include <utility>

namespace dash {

bool dag_longest_path(int n_nodes, const double* w, int n_edges, const int* src, const int* dst,
                      const double* lat, double* start, double* finish) {
  std::vector<int> head(n_nodes, -1), next(n_edges), indeg(n_nodes, 0);
  for (int e = 0; e < n_edges; ++e) {
    next[e] = head[src[e]];
    head[src[e]] = e;
    ++indeg[dst[e]];
  }
  std::vector<int> order;
  order.reserve(n_nodes);
  for (int v = 0; v < n_nodes; ++v) {
    start[v] = 0.0;
    if (!indeg[v]) order.push_back(v);
  }
  for (size_t k = 0; k < order.size(); ++k) {
    const int u = order[k];
    finish[u] = start[u] + w[u];
    for (int e = head[u]; e >= 0; e = next[e]) {
      const int v = dst[e];
      start[v] = std::max(start[v], finish[u] + lat[e]);
      if (--indeg[v] == 0) order.push_back(v);
    }
  }
  return (int)order.size() == n_nodes;
}

bool dag_predict(const Tables& t, int heads, int slots, const double cost[4], DagResult& out,
                 bool unit_major) {
  const int n = t.n, U = t.units(), I = t.items();
  if (heads < 1 || slots < 1) return false;
  if (U == 0) {  // nothing to run (every pair masked)
    out = DagResult();
    return true;
  }
  const double c_full = cost[0], c_diag = cost[1], r = cost[2], hlat = cost[3];
  // partial pairs (the causal diagonal; window or block edges) cost c_diag
  auto ccost = [&](int i) { return t.partial[(size_t)t.q[i] * t.n + t.kv[i]] ? c_diag : c_full; };

  // rank predecessor of every item within one head (-1 for the first / atomic)
  std::vector<int> pos((size_t)n * n, -1), pred(I, -1);
  for (int i = 0; i < I; ++i) pos[(size_t)t.q[i] * n + t.kv[i]] = i;
  if (t.ordered()) {
    for (int q = 0; q < n; ++q) {
      std::vector<int> by_rank(n, -1);
      for (int kv = 0; kv < n; ++kv) {
        const int rk = t.rank[(size_t)q * n + kv];
        if (rk >= 0) by_rank[rk] = pos[(size_t)q * n + kv];
      }
      for (int rk = 1; rk < n && by_rank[rk] >= 0; ++rk) pred[by_rank[rk]] = by_rank[rk - 1];
    }
  }

  const long total_units = (long)U * heads;
  // global unit order: head-major (g = head * U + unit) or, for the dynamic
  // policy on request, unit-major (g = unit * heads + head)
  const bool um = unit_major && !t.needs_static();
  auto head_of = [&](long g) { return (int)(um ? g % heads : g / U); };
  auto unit_of = [&](long g) { return (int)(um ? g / heads : g % U); };
  std::vector<int> slot_of(total_units);
  if (t.needs_static()) {
    if (U > slots) return false;
    const int p_eff = (slots / U) * U;
    for (long g = 0; g < total_units; ++g) slot_of[g] = (int)(g % p_eff);
  } else {
    // first free slot, ties to the lowest index; times follow the model
    typedef std::pair<double, int> Ev;
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> freeq;
    for (int s = 0; s < slots; ++s) freeq.push(Ev(0.0, s));
    std::vector<double> r_fin((size_t)I * heads, 0.0);
    for (long g = 0; g < total_units; ++g) {
      const Ev ev = freeq.top();
      freeq.pop();
      slot_of[g] = ev.second;
      const int hd = head_of(g), u = unit_of(g);
      double tnow = ev.first;
      for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i) {
        double tr = tnow + ccost(i);
        if (pred[i] >= 0) tr = std::max(tr, r_fin[(size_t)hd * I + pred[i]] + hlat);
        tnow = tr + r;
        r_fin[(size_t)hd * I + i] = tnow;
      }
      freeq.push(Ev(tnow, ev.second));
    }
  }

  // explicit graph: node 2*gi = C, 2*gi+1 = R, gi = head*I + i
  const long nodes = 2L * I * heads;
  std::vector<double> wt(nodes);
  std::vector<int> src, dst;
  std::vector<double> lat;
  for (int hd = 0; hd < heads; ++hd)
    for (int i = 0; i < I; ++i) {
      const long gi = (long)hd * I + i;
      wt[2 * gi] = ccost(i);
      wt[2 * gi + 1] = r;
      src.push_back((int)(2 * gi));
      dst.push_back((int)(2 * gi + 1));
      lat.push_back(0.0);
      if (pred[i] >= 0) {
        src.push_back((int)(2 * ((long)hd * I + pred[i]) + 1));
        dst.push_back((int)(2 * gi + 1));
        lat.push_back(hlat);
      }
    }
  std::vector<long> last_r(slots, -1);
  for (long g = 0; g < total_units; ++g) {
    const int hd = head_of(g), u = unit_of(g);
    const int a = t.unit_off[u], b = t.unit_off[u + 1];
    if (a == b) continue;
    for (int i = a + 1; i < b; ++i) {
      src.push_back((int)(2 * ((long)hd * I + i - 1) + 1));
      dst.push_back((int)(2 * ((long)hd * I + i)));
      lat.push_back(0.0);
    }
    const int s = slot_of[g];
    if (last_r[s] >= 0) {
      src.push_back((int)last_r[s]);
      dst.push_back((int)(2 * ((long)hd * I + a)));
      lat.push_back(0.0);
    }
    last_r[s] = 2 * ((long)hd * I + b - 1) + 1;
  }
  std::vector<double> st(nodes), fin(nodes);
  if (!dag_longest_path((int)nodes, wt.data(), (int)src.size(), src.data(), dst.data(), lat.data(),
                        st.data(), fin.data()))
    return false;

  DagResult res;
  std::vector<double> busy(slots, 0.0);
  double longest_unit = 0.0;
  for (long v = 0; v < nodes; ++v) res.makespan = std::max(res.makespan, fin[v]);
  for (long gi = 0; gi < (long)I * heads; ++gi) res.total_wait += st[2 * gi + 1] - fin[2 * gi];
  for (long g = 0; g < total_units; ++g) {
    const int u = unit_of(g);
    double len = 0.0;
    for (int i = t.unit_off[u]; i < t.unit_off[u + 1]; ++i) len += ccost(i) + r;
    busy[slot_of[g]] += len;
    longest_unit = std::max(longest_unit, len);
  }
  double work = 0.0;
  for (int s = 0; s < slots; ++s) {
    work += busy[s];
    res.max_slot_idle = std::max(res.max_slot_idle, res.makespan - busy[s]);
  }
  res.lower_bound = std::max(work / slots, longest_unit);
  out = res;
  return true;
}

}  // namespace dash
