// Host-side launch interface of the HIP kernels (private to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

// Largest number of items (KV tile x Q block pairs) in one unit's work list;
// the backward stages a unit's list in LDS.
constexpr int kMaxUnitItems = 1024;

// Arguments of the persistent backward kernel.  All pointers are device
// pointers.  Per-head tensors are indexed by head = b*H + h.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* lse2;      // [BH, N] LSE * log2(e) (two-stage pipeline only)
  const float* delta;
  void* dq;               // final dQ (ordered schedules write it directly)
  void* dk;
  void* dv;
  float* dq_accum;        // [BH, N, d] fp32 (zeroed before the launch only for atomic)
  uint32_t* counters;     // [BH, N / BR, waves] order counters, zeroed
  uint32_t* header;       // [0] status word, [1] work counter; zeroed
  const int* unit_off;    // [units_per_head + 1]
  const int2* items;      // {kv | q << 16, rank | partial << 29 | last << 30} per item
  int N;
  int n_tiles;            // N / BC
  int mask_lo, mask_hi;   // pairs flagged partial: key j visible to query i iff lo <= i - j <= hi
  int units_per_head;
  int total_units;        // units_per_head * BH
  int p_eff;              // static policy: workgroups that take units
  int dynamic;            // 1: take units from the work counter
  int unit_major;         // dynamic only: 1 = unit lu of every head in turn, 0 = head by head
  int timed_slots;        // dynamic timed shift: slots per head it was timed on (0: none);
                          // a group of W workgroups with h heads needs W >= (slots-1)h + 1
  int xcd_mode;           // 0 device-wide; XCD-local groups when they fit with
                          // 1: L2-coherent, 2: device-coherent accumulator
  float scale;            // softmax scale s
  float scale_log2;       // s * log2(e)
  uint32_t spin_limit;
  uint32_t jitter_seed;
  int poison_q;
  float* partials;        // debug: [BH, n_tiles, N, d] or null
  uint64_t* wait_stats;   // debug: [grid, waves, 4] or null
  uint64_t* phase_stats;  // debug: [grid, waves, 16] or null
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;
  int BH;
  float scale_log2;
  int mask_lo, mask_hi;   // masked kernels: key j visible to query i iff lo <= i - j <= hi
  const uint8_t* live;    // or null; else tile pair (i / tile, j / tile) must be live too
  int n_tiles;            // N / tile
  int tile;
};

// dtype: 0 = fp32, 1 = bf16.  Returns hipSuccess or the launch error.
// masked: some pairs carry the partial flag (elements hidden by mask_lo/hi).
hipError_t launch_bwd(int dtype, int d, bool masked, bool ordered, const BwdArgs& a, int grid,
                      hipStream_t stream);
// Largest grid of the backward kernel whose workgroups are all resident.
hipError_t bwd_max_coresident(int dtype, int d, bool masked, bool ordered, int* blocks);

// Wave-pair layout of the backward (bf16, d = 128 only): same arguments,
// 512 threads per workgroup.
hipError_t launch_bwd_pair(bool masked, bool ordered, const BwdArgs& a, int grid,
                           hipStream_t stream);
hipError_t bwd_pair_max_coresident(bool masked, bool ordered, int* blocks);
// Two-stage pipeline layout of the backward (bf16, d = 128 or 64): same
// arguments plus the head dim, 512 threads per workgroup.
hipError_t launch_bwd_pipe(int d, bool masked, bool ordered, const BwdArgs& a, int grid,
                           hipStream_t stream);
hipError_t bwd_pipe_max_coresident(int d, bool masked, bool ordered, int* blocks);
// Tile sizes of the backward kernel: KV tile (BC) and Q sub-tile (BR).
void bwd_tiles(int dtype, int d, int* bc, int* br);
// Waves per workgroup of the backward kernel (one order counter each).
int bwd_waves(int dtype, int d);

hipError_t launch_fwd(int dtype, int d, bool masked, const FwdArgs& a, hipStream_t stream);

// Size of the built-in scratch array of the allocation-free backward.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress).
hipError_t noalloc_scratch(void** out);

hipError_t launch_preprocess(int dtype, int d, const void* o, const void* dout, float* delta,
                             long rows, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, size_t n_words, hipStream_t stream);

// Workspace prologue of the backward: clear [clear, clear + clear_words)
// and [clear2, clear2 + clear2_words), and, when n > 0, write the plain
// mask's schedule tables (closed forms, plain_tables.hpp) for `sched`:
// unit_off[0 .. units] and item[0 .. items).  Both clears are 16-byte
// aligned multiples of 4 words.
struct PrologueArgs {
  uint32_t* clear = nullptr;
  size_t clear_words = 0;
  uint32_t* clear2 = nullptr;
  size_t clear2_words = 0;
  int n = 0, causal = 0, sched = 0, units = 0;
  long items = 0;
  int* unit_off = nullptr;
  int2* item = nullptr;
  // lse2[i] = lse[i] * log2(e), rounded once, for i < lse_count
  const float* lse = nullptr;
  float* lse2 = nullptr;
  size_t lse_count = 0;
};
hipError_t launch_bwd_prologue(const PrologueArgs& a, hipStream_t stream);
// Zero rows [t * rows, t * rows + rows) of every head of a [BH, N, d] tensor
// for each tile t in tiles[0..count) (a device array).
hipError_t launch_zero_tiles(int dtype, void* base, const int* tiles, int count, int rows, int d,
                             int N, int BH, hipStream_t stream);
hipError_t launch_dq_convert(int dtype, const float* acc, void* dq, float scale, size_t n,
                             hipStream_t stream);
hipError_t launch_litmus(int contributors, int len, const int* turn, const float* values,
                         float* acc, uint32_t* counter, uint32_t* status, uint32_t spin_limit,
                         hipStream_t stream);

}  // namespace dash
