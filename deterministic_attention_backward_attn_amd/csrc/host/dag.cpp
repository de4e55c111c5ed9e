// DAG critical-path calculator: see dag.hpp for the model.
#include "dag.hpp"

#include <algorithm>
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
    // Event simulation of the work counter: a slot that becomes free takes
    // the next unit (free slots in time order, ties to the lowest index);
    // an item whose rank predecessor has not finished waits for it, also
    // when that predecessor's unit was handed out later (timed shift).
    typedef std::pair<double, int> Ev;  // (time the slot's next step starts, slot)
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> evq;
    std::vector<long> cur(slots, -1);   // global unit on the slot, -1 when free
    std::vector<int> pos_in(slots, 0);  // next item of that unit
    std::vector<double> r_fin((size_t)I * heads, -1.0);
    std::vector<int> waiter((size_t)I * heads, -1);  // slot blocked on this item
    std::vector<double> ready((size_t)I * heads, 0.0);  // start of a blocked item
    long next_unit = 0, done_units = 0;
    for (int s = 0; s < slots; ++s) evq.push(Ev(0.0, s));
    // run slots' items until each blocks or frees; an item that finishes
    // hands its blocked successor's slot to the same loop (times only grow:
    // every slot resumed here runs at or after the event being handled)
    std::vector<std::pair<int, double>> work;
    auto advance = [&](int s0, double t0) {
      work.push_back(std::make_pair(s0, t0));
      while (!work.empty()) {
        const int s = work.back().first;
        double tnow = work.back().second;
        work.pop_back();
        for (;;) {
          if (cur[s] < 0) {
            evq.push(Ev(tnow, s));  // free: takes a unit when its turn comes
            break;
          }
          const long g = cur[s];
          const int hd = head_of(g), u = unit_of(g);
          const size_t gi = (size_t)hd * I + t.unit_off[u] + pos_in[s];
          const int p = pred[t.unit_off[u] + pos_in[s]];
          if (p >= 0 && r_fin[(size_t)hd * I + p] < 0.0) {
            waiter[(size_t)hd * I + p] = s;
            ready[gi] = tnow;
            break;
          }
          double tr = tnow + ccost((int)(gi - (size_t)hd * I));
          if (p >= 0) tr = std::max(tr, r_fin[(size_t)hd * I + p] + hlat);
          tnow = tr + r;
          r_fin[gi] = tnow;
          if (++pos_in[s] == t.unit_off[u + 1] - t.unit_off[u]) {
            cur[s] = -1;
            ++done_units;
          }
          const int w = waiter[gi];
          if (w >= 0) {
            waiter[gi] = -1;
            const size_t wi = (size_t)head_of(cur[w]) * I + t.unit_off[unit_of(cur[w])] + pos_in[w];
            work.push_back(std::make_pair(w, ready[wi]));
          }
        }
      }
    };
    while (!evq.empty()) {
      const Ev ev = evq.top();
      evq.pop();
      const int s = ev.second;
      if (cur[s] >= 0) continue;  // stale
      if (next_unit >= total_units) continue;
      cur[s] = next_unit;
      pos_in[s] = 0;
      slot_of[next_unit++] = s;
      advance(s, ev.first);
    }
    if (done_units != total_units) return false;  // the counter would deadlock
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
