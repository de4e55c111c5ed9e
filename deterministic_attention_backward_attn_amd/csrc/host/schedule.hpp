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

// Which tile pairs exist.  A plain mask is the full square or the causal
// triangle, where the pages' constructions apply; otherwise the pairs come
// from a sliding window and/or a block mask (the summary lists block-sparse
// and other special masks as needing schedule extensions).  A pair is live
// when some (query, key) in it is visible and partial when it is live but
// some pair in it is hidden (the kernel then masks elements).
struct TileMask {
  int n = 0;
  bool causal = false;
  bool plain = true;
  std::vector<uint8_t> live;     // [q * n + kv]
  std::vector<uint8_t> partial;  // [q * n + kv]
  bool any_partial() const;
};

TileMask plain_mask(int n, bool causal);

// Element rule: key j visible to query i when (not causal or j <= i), the
// window (if > 0) holds (causal: i - j < window; else |i - j| < window) and
// the block mask (if any; row = query block, bt tiles per block side) is
// nonzero.  `tile` is the tile side in rows.  A window that covers the
// whole sequence and no block mask gives the plain mask.
TileMask make_mask(int n, int tile, bool causal, int window, const uint8_t* block, int bt);

// Element bounds of the same rule as a range of i - j: lo <= i - j <= hi
// (+-2^30 where unbounded).
void mask_bounds(bool causal, int window, int* lo, int* hi);

struct Tables {
  int n = 0;
  bool causal = false;
  Sched sched = Sched::Naive;
  std::vector<uint8_t> live;     // [n * n] by [q * n + kv]
  std::vector<uint8_t> partial;  // [n * n]
  std::vector<int> unit_off;  // [units + 1]
  std::vector<int> kv;        // [items]
  std::vector<int> q;         // [items]
  std::vector<int> step;      // [items] lockstep step of each item (SHIFT), else empty
  std::vector<int> rank;      // [n * n], -1 where absent or unordered
  // Units must be taken in head-aligned rounds (some wait points to a later
  // unit): the pages' SHIFT on the full and causal masks.
  bool static_policy = false;
  // SHIFT on a window or block mask (timed shift): the units were timed on
  // this many workgroup slots per head; see build_tables.  0 otherwise.
  int slots_per_head = 0;
  std::vector<int> unit_start;  // timed shift: the step at which each unit took a slot
  int units() const { return (int)unit_off.size() - 1; }
  int items() const { return (int)kv.size(); }
  bool ordered() const { return sched != Sched::Atomic; }
  bool needs_static() const { return static_policy; }
  bool timed() const { return slots_per_head > 0; }
};

// Returns false when the schedule is undefined for (n, causal): symmetric
// shift with odd n > 1.
bool build_tables(int n, bool causal, Sched s, Tables& t);
// Any mask.  SHIFT on a plain mask is the pages' cyclic / symmetric shift.
// On any other mask it is a timed shift for `slots` workgroups per head
// (the summary names block-sparse masks as needing schedule extensions):
// one unit per KV tile with live pairs, started longest first (ties: lower
// KV tile) whenever one of the `slots` slots is free; at every step each
// running unit, in start order, takes the remaining Q block of its own
// that no other unit took at this step and that comes first cyclically
// from its own diagonal (smallest (q - kv) mod n), or idles for the step
// when every one is taken.  Items run in step order, units in start order,
// and a block's dQ order is by step, so concurrent units never meet on a
// block.  The tables run deadlock-free from a work counter on W
// workgroups shared by h heads, in any interleaving of the heads' units,
// when W >= (slots - 1) * h + 1 (timed_slots).
bool build_tables(const TileMask& m, Sched s, Tables& t, int slots = 1);

// Slots per head of a timed shift for a launch on `maxco` co-resident
// workgroups, `heads` heads of `units` units each: the largest count that
// is deadlock-free both in 8 XCD groups of maxco / 8 workgroups (each with
// ceil(heads / 8) heads) and device-wide (min(maxco, heads * units)
// workgroups, all heads), at most `units`, at least 1.
int timed_slots(int maxco, long heads, int units);

// Workgroups that a timed shift of `slots` slots per head needs for h heads.
inline long timed_need(int slots, long h) { return (long)(slots - 1) * h + 1; }

// Structural checks: every live pair exactly once, each KV tile's items
// contiguous in one unit, every rank row a permutation, and for the
// dynamic policy either every wait pointing to an earlier unit or (timed
// shift) the timing certificate: steps increasing within a unit and
// distinct within a Q block, dQ orders by step, units listed in start
// order, no item before its unit's start, and at most slots_per_head units
// between their start and their last step at any step.  Returns an empty string when valid, else a
// description.
const char* validate_tables(const Tables& t);

}  // namespace dash
