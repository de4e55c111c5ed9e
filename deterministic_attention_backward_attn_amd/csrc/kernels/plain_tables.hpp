// Closed-form schedule tables for the plain masks (full square, causal
// triangle), usable on the host and on the device.
//
// The backward writes these tables into the caller's workspace with a
// kernel at every launch, so the plain masks need no host-to-device copy
// and no library-owned device memory.  The host builds the same tables with
// the general schedule builder and checks, once per (n, mask, schedule),
// that both agree item for item before the first launch.
//
// Item encoding (int2): x = kv | q << 16; y = rank | partial << 29 |
// last << 30 (rank and last for ordered schedules only).  Items of unit u
// are [unit_off(u), unit_off(u + 1)).
//
// Schedules (DASH explainer, "Technisches Resuemee" 2.2 A and B):
//   NAIVE / ATOMIC  unit kv visits its live Q blocks ascending
//   DESCENDING      unit kv visits them descending (same dQ order as NAIVE)
//   SHIFT, full     unit i visits Q block (i + t) mod n at step t
//   SHIFT, causal   symmetric shift: unit w runs KV tile w, then n-1-w,
//                   n+1 items: a dense phase over the lower-left square,
//                   then the two folded triangles as n/2+1 super-rows
// dQ order: ascending kv for NAIVE and DESCENDING, by step for SHIFT.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {
namespace plain {

enum : int { kAtomic = 0, kNaive = 1, kDescending = 2, kShift = 3 };

__host__ __device__ inline int pmod(int a, int m) {
  const int r = a % m;
  return r < 0 ? r + m : r;
}

// Whether (n, causal, schedule) has a closed form here: symmetric shift
// needs n even (or n == 1).
__host__ __device__ inline bool defined(int n, bool causal, int sched) {
  return n >= 1 && sched >= kAtomic && sched <= kShift &&
         !(sched == kShift && causal && n > 1 && (n & 1));
}

__host__ __device__ inline int units(int n, bool causal, int sched) {
  return (sched == kShift && causal && n > 1) ? n / 2 : n;
}

__host__ __device__ inline long items(int n, bool causal) {
  return causal ? (long)n * (n + 1) / 2 : (long)n * n;
}

// First item of unit u (u == units() gives the item count).
__host__ __device__ inline long unit_off(int n, bool causal, int sched, int u) {
  if (sched == kShift && causal && n > 1) return (long)u * (n + 1);
  if (!causal) return (long)u * n;
  // unit kv holds Q blocks kv .. n-1
  return (long)u * n - (long)u * (u - 1) / 2;
}

// Global step of (kv, q) in the symmetric shift (n even, kv <= q): phase 1
// steps 0 .. n/2-1 over the square Q blocks n/2.., KV tiles ..n/2-1; phase 2
// steps n/2 .. n over the super-rows.
__host__ __device__ inline int sym_step(int n, int kv, int q) {
  const int h = n / 2;
  if (kv < h) {
    if (q >= h) return pmod(q - h - kv, h);
    return h + pmod(q - kv, h + 1);  // upper row q is super-row q
  }
  const int w = n - 1 - kv;
  const int k = (q == n - 1) ? h : n - 2 - q;  // lower row q
  return h + pmod(k - w, h + 1);
}

// Item i (global index over the head's units in order).
__host__ __device__ inline void item(int n, bool causal, int sched, long i, int* kv, int* q,
                                     int* rank, bool* last) {
  int a = 0, b = 0, r = 0, cnt = 0;
  if (sched == kShift && causal && n > 1) {
    const int h = n / 2;
    const int w = (int)(i / (n + 1));
    const int j = (int)(i % (n + 1));
    if (j < h) {
      a = w;
      b = h + (w + j) % h;
    } else {
      const int k = (w + j - h) % (h + 1);
      if (k <= h - 2) {
        if (w <= k) { a = w; b = k; }
        else { a = n - 1 - w; b = n - 2 - k; }
      } else if (k == h - 1) {
        a = w; b = h - 1;
      } else {
        a = n - 1 - w; b = n - 1;
      }
    }
    // rank: contributors of Q block b (KV tiles 0..b) reached at an earlier step
    const int s = sym_step(n, a, b);
    for (int x = 0; x <= b; ++x) r += sym_step(n, x, b) < s ? 1 : 0;
    cnt = b + 1;
  } else if (sched == kShift) {  // full mask (or a single tile)
    const int u = (int)(i / n);
    const int t = (int)(i % n);
    a = u;
    b = (u + t) % n;
    r = t;
    cnt = n;
  } else {
    // NAIVE, DESCENDING, ATOMIC: unit kv = u
    int u = 0;
    if (!causal) {
      u = (int)(i / n);
    } else {
      // largest u with unit_off(u) <= i
      int lo = 0, hi = n - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (unit_off(n, true, sched, mid) <= i) lo = mid;
        else hi = mid - 1;
      }
      u = lo;
    }
    const int j = (int)(i - unit_off(n, causal, sched, u));
    const int first = causal ? u : 0;
    a = u;
    b = sched == kDescending ? n - 1 - j : first + j;
    r = u;  // ascending kv among the block's contributors 0 .. (causal ? b : n-1)
    cnt = causal ? b + 1 : n;
  }
  *kv = a;
  *q = b;
  *rank = r;
  *last = r == cnt - 1;
}

__host__ __device__ inline int2 encode(int n, bool causal, int sched, long i) {
  int kv = 0, q = 0, rank = 0;
  bool last = false;
  item(n, causal, sched, i, &kv, &q, &rank, &last);
  int2 e;
  e.x = kv | (q << 16);
  e.y = (causal && kv == q) ? (1 << 29) : 0;
  if (sched != kAtomic) e.y |= rank | (last ? (1 << 30) : 0);
  return e;
}

}  // namespace plain
}  // namespace dash
