// Unit placement of the persistent backward kernels (device side).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace dash {

// Where a workgroup takes its units from.
struct Placement {
  int grp;        // XCD group of this workgroup (0 when device-wide)
  int n_grp;      // number of groups
  int li;         // index of this workgroup within its group
  int W;          // workgroups in its group
  bool grouped;   // units come from the group's own list
  bool xl;        // ... and the accumulator is coherent within the group's L2
};

// XCD groups: every workgroup reads the XCD it runs on, a census (all
// workgroups are resident: cooperative launch) counts workgroups per XCD,
// and the heads are dealt round-robin to the XCDs present.  All units of a
// head then run on one XCD, so its ordered dQ hand-offs stay inside that
// XCD's L2 (L2-coherent accumulator accesses) and its Q/dO tiles are reused
// from that L2.  A static schedule needs a whole head resident, and a timed
// shift (slots s per head) needs (s - 1) * h + 1 workgroups for a group of
// h heads, so if some XCD has fewer, every workgroup falls back to one
// device-wide group with device-coherent accesses (the host sized the
// timed shift for that case too).
// Header words: [0] status, [1] device work counter, [2] census arrivals,
// [4..19] workgroups per XCD, [20..35] work counter per XCD group.
// Every thread of the workgroup must call this (it contains a barrier).
__device__ __forceinline__ Placement place_units(const BwdArgs& a, int tid, int* sPlace) {
  Placement p{0, 1, (int)blockIdx.x, (int)gridDim.x, false, false};
  if (!a.xcd_mode) return p;
  if (tid == 0) {
    uint32_t* status = a.header;
    const uint32_t x = xcc_id();
    const uint32_t mine = __hip_atomic_fetch_add(&a.header[4 + x], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&a.header[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_counter(&a.header[2], gridDim.x, status, a.spin_limit);
    int active = 0, my_grp = 0, fits = 1, fewest = 1 << 30;
    for (uint32_t k = 0; k < 16; ++k) {
      const uint32_t c = load_relaxed_agent(&a.header[4 + k]);
      if (c == 0) continue;
      if (k == x) my_grp = active;
      if (!a.dynamic && (int)c < a.units_per_head) fits = 0;
      fewest = (int)c < fewest ? (int)c : fewest;
      ++active;
    }
    if (a.dynamic && a.timed_slots > 0) {
      const int bh = a.total_units / a.units_per_head;
      const int hg = (bh + active - 1) / active;  // most heads of one group
      if ((long)(a.timed_slots - 1) * hg + 1 > (long)fewest) fits = 0;
    }
    sPlace[0] = my_grp;
    sPlace[1] = active;
    sPlace[2] = (int)mine;
    sPlace[3] = (int)load_relaxed_agent(&a.header[4 + x]);
    sPlace[4] = fits && load_relaxed_agent(status) == 0u;
  }
  __syncthreads();
  if (sPlace[4]) {
    p.grouped = true;
    p.xl = a.xcd_mode == 1;
    p.grp = sPlace[0];
    p.n_grp = sPlace[1];
    p.li = sPlace[2];
    p.W = sPlace[3];
  }
  return p;
}

}  // namespace dash
