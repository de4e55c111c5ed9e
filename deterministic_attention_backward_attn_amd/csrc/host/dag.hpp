// DAG critical-path calculator (plain C++).
//
// The DASH explainer ("Technisches Resuemee" 2.1) models the deterministic
// backward as a DAG: compute nodes (one KV tile meeting one Q block) and
// reduction nodes (adding that dQ partial), with data edges and the
// mandatory accumulation-order edges, one KV tile's work forming an
// unbroken chain on one processor; the objective is the critical-path
// length.  Here: P persistent workgroup slots, item nodes C (c_full or
// c_diag) -> R (r), unit chains, slot chains, and order edges R -> R with
// hand-off latency h.  Units go to slots by the kernel's own policy:
// dynamic (first free slot, head-major or unit-major order; an add may wait
// for a unit handed out later, as in the timed shift) or static
// head-aligned rounds.
#pragma once

#include <cstdint>
#include <vector>

#include "schedule.hpp"

namespace dash {

struct DagResult {
  double makespan = 0, total_wait = 0, max_slot_idle = 0, lower_bound = 0;
};

// Longest path of a general DAG.  Returns false on a cycle.
bool dag_longest_path(int n_nodes, const double* w, int n_edges, const int* src, const int* dst,
                      const double* lat, double* start, double* finish);

// Returns false if the policy cannot run these tables on `slots` slots
// (static policy with fewer slots than units per head) or on a cycle.
// unit_major: the dynamic policy takes unit 0 of every head, then unit 1 of
// every head, ... (default: head after head).
bool dag_predict(const Tables& t, int heads, int slots, const double cost[4], DagResult& out,
                 bool unit_major = false);

}  // namespace dash
