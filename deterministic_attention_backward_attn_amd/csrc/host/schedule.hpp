// Schedule layer: per-head work lists and dQ rank tables (plain C++).
//
// A head is tiled square: n KV tiles and n Q blocks of the same width.  An
// item (kv, q) is one KV tile meeting one Q block (causal: only q >= kv).
// A unit is what one workgroup runs without interruption; its items are
// grouped by KV tile so the tile's dK/dV stay in registers (DASH explainer,
// "Technisches Resuemee" 2.1).  rank[q*n + kv] is kv's position in Q block
// q's dQ accumulation order.
#pragma once

#include <cstdint>
#include <vector>

namespace dash {

enum class Sched : int { Atomic = 0, Naive = 1, Descending = 2, Shift = 3 };

struct Tables {
  int n = 0;
  bool causal = false;
  Sched sched = Sched::Naive;
  std::vector<int> unit_off;  // [units + 1]
  std::vector<int> kv;        // [items]
  std::vector<int> q;         // [items]
  std::vector<int> rank;      // [n * n], -1 where absent or unordered
  int units() const { return (int)unit_off.size() - 1; }
  int items() const { return (int)kv.size(); }
  bool ordered() const { return sched != Sched::Atomic; }
  // Units must be taken in head-aligned rounds (waits point to later units).
  bool needs_static() const { return sched == Sched::Shift; }
};

// Returns false when the schedule is undefined for (n, causal): symmetric
// shift with odd n > 1.
bool build_tables(int n, bool causal, Sched s, Tables& t);

// Structural checks: every live pair exactly once, each KV tile's items
// contiguous in one unit, every rank row a permutation, and (for the
// dynamic policy) every wait pointing to an earlier unit.  Returns an
// empty string when valid, else a description.
const char* validate_tables(const Tables& t);

}  // namespace dash
