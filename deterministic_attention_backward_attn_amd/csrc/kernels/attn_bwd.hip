// Persistent deterministic attention backward for gfx950.
//
// One workgroup owns one KV tile (BC rows) at a time and keeps that tile's
// dK and dV accumulators in registers for as long as it works on it (the
// DASH explainer, "Technisches Resuemee" 2.1: one KV tile's operations run
// as an uninterrupted chain on one processor with register-resident
// accumulation).  For every Q block in its schedule it recomputes, per Q
// sub-tile of BR rows:
//   S   = Q K^T                (MFMA; K held in registers)
//   P   = exp(s S - LSE)       (exactly 0 where the mask hides a key)
//   dP  = dO V^T               (MFMA; V held in registers)
//   dS  = P (dP - delta)
//   dV += P^T dO ; dK += dS^T Q  (MFMA, accumulators in registers)
//   dQ_part = dS K             (MFMA, dS staged through LDS)
// and adds dQ_part into the fp32 accumulator of that Q sub-tile.
//
// Ordered schedules add in a fixed order (explainer section 1: a fixed
// accumulation order for dQ): each wave owns the same dQ output columns in
// every workgroup, so wave w of the contributor ranked r waits until the
// sub-tile's counter for wave w reads r, reads the accumulator, adds its
// partial, writes it back and sets the counter to r + 1.  The first
// contributor writes without reading; the last one writes the final,
// scaled dQ in the output dtype instead of the accumulator.  The counters
// are accessed with device-coherent loads and stores (the cache policy of
// device-scope atomics); the accumulator too, or with L2-coherent ones when
// every contributor of a head runs on one XCD (then this CU's L1 is
// invalidated right before each accumulator read).  A wave's stores complete
// before it advances the counter, so no cache-wide write-back is needed.  The add for sub-tile g runs during sub-tile g+1's products, so its
// memory latency hides behind MFMA work.  The atomic schedule adds with
// unordered fp32 atomics instead (non-deterministic reference).
//
// The workgroups form a persistent grid: each takes units (work lists from
// the schedule tables) either from a work counter in increasing order
// (schedules whose waits point only to earlier units, and the timed shift of
// window and block masks, whose waits point only to units that reached the
// block earlier in its simulated timing, run on enough workgroups) or in
// head-aligned rounds (the pages' shift, whose waits point to other units of
// the same head, all of which are then resident).
//
// Operand placement (see common.hpp for the MFMA layouts):
//   S and dP are computed as (Q-rows x KV-cols): the accumulators hold KV on
//   lanes and Q rows in registers and serve directly as the A operand of
//   dV += P^T dO and dK += dS^T Q.  Those products need dO and Q with Q rows
//   in the K slots; bf16 reads them from the row-major LDS tiles with the
//   transposing LDS read (ds_read_b64_tr_b16), fp32 with element reads.
//   dQ = dS K needs dS with Q rows on lanes: dS goes to LDS as dS^T
//   ([kv][q], 8-byte writes) and comes back through the transposing read;
//   K^T fragments (d on lanes) are built once per KV tile the same way.
#include "common.hpp"
#include "launch.hpp"
#include "placement.hpp"

namespace dash {

// phases of a sub-tile timed by the phase-timer test hook
constexpr int kPhases = 11;

template <typename T, int D, int BC, int BR, bool MASKED, bool ORDERED, bool DEBUG>
__global__ void __launch_bounds__(BC * 2, 1) bwd_kernel(BwdArgs a) {
  using E = Elt<T>;
  using frag = typename E::frag;
  constexpr int NW = BC / 32;          // waves; wave w owns KV rows [32w, 32w+32)
  constexpr int NT = NW * 64;
  constexpr int RHO = BC / BR;         // Q sub-tiles per Q block
  constexpr int KPL = E::KPL;
  constexpr int KSTEP = E::KSTEP;
  constexpr int VEC = E::VEC;          // elements per 16-byte access
  constexpr int DK = D / KSTEP;        // MFMA steps over d
  constexpr int KK = BC / KSTEP;       // MFMA steps over a KV tile
  constexpr int MT = BR / 32;          // 32-row tiles of a Q sub-tile
  constexpr int NTD = D / 32;          // 32-column tiles over d
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr bool SWZ = sizeof(T) == 2;  // bf16: swizzled sQ, sdO, sK
  constexpr int LQ = SWZ ? D : D + PAD;  // row stride of sQ, sdO, sK ([row][d])
  // row stride of sdSt ([kv][q]); bf16 with 32-column rows pads by 4
  // elements, which keeps the 8-byte writes of 32 rows on distinct banks
  constexpr int LS = (SWZ && BR == 32) ? BR + 4 : BR + PAD;
  constexpr int CPT = BR * D / VEC / NT;  // 16-byte chunks per thread per tensor
  // dQ output tiles of a wave: CPW column tiles x RPW row tiles
  constexpr int CPW = NTD >= NW ? NTD / NW : 1;
  constexpr int WPC = NW > NTD ? NW / NTD : 1;  // waves sharing a column tile
  constexpr int RPW = MT / WPC;
  constexpr int QT = CPW * RPW;
  static_assert(BC % BR == 0 && BR % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(NTD % NW == 0 || NW % NTD == 0, "dQ columns must split over waves");
  static_assert(MT % WPC == 0, "dQ rows must split over waves");
  static_assert(CPT * VEC * NT == BR * D, "sub-tile load must split evenly");
  static_assert(NT >= 2 * BR, "LSE/delta staging needs 2*BR threads");

  // Double-buffered Q / dO / LSE / delta sub-tiles and dS^T: sub-tile g reads
  // buffer g%2 while the next one is staged into the other, so a sub-tile
  // needs one workgroup barrier.
  __shared__ __align__(16) T sQ[2][BR * LQ];
  __shared__ __align__(16) T sdO[2][BR * LQ];
  __shared__ __align__(16) T sdSt[2][BC * LS];
  __shared__ __align__(16) T sK[BC * LQ];
  __shared__ __align__(16) float sLSE[2][BR];
  __shared__ __align__(16) float sDel[2][BR];
  __shared__ int2 sItems[kMaxUnitItems];
  // per-wave staging of a dQ partial, row-major [32 rows][32 + 4 floats], so
  // that each 16-byte accumulator access of a lane group covers whole rows
  // (rows of 32 floats, 16-byte chunk c of row r at chunk c ^ ((r/2)%8), so
  // that 32 rows of one chunk and 8 whole rows each spread over all banks)
  constexpr int LR = 32;
  __shared__ __align__(16) float sRow[ORDERED ? NW : 1][ORDERED ? QT * 32 * LR : 4];
  __shared__ int sUnit;
  __shared__ int sPlace[5];
  // element offset of (row, col) in sQ, sdO, sK
  const auto qix = [](int r, int c) {
    if constexpr (SWZ) return r * LQ + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7);
    else return r * LQ + c;
  };
  const auto six = [](int r, int c) { return r * LS + c; };  // sdSt
  const auto rix = [](int r, int c) { return r * LR + (((c >> 2) ^ ((r >> 1) & 7)) << 2) + (c & 3); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int j16 = lane & 15;
  const int gcol = 16 * ((lane >> 4) & 1);  // column offset of this lane's 16-lane group
  const int N = a.N;
  const int n_sub = N / BR;
  uint32_t* status = a.header;
  const uint32_t spin_limit = a.spin_limit;
  const int col0 = w % NTD;            // first dQ column tile of this wave
  const int row0 = NW > NTD ? w / NTD : 0;

  // diagnostics (lane 0 of each wave): cycles in ordered waits, waits, waits
  // that had to poll more than once, cycles of the whole unit loop
  uint64_t st_wait = 0, st_waits = 0, st_spun = 0;
  const uint64_t st_t0 = (DEBUG && a.wait_stats) ? (uint64_t)clock64() : 0;
  // phase timer (test hook): lane 0 of each wave adds the shader-clock
  // cycles since the previous mark to the phase that just ended
  uint64_t ph[kPhases] = {};
  uint64_t ph_t = (DEBUG && a.phase_stats) ? (uint64_t)clock64() : 0;
  const uint64_t ph_t0 = ph_t;
#define PHASE(k)                                                   \
  if (DEBUG && a.phase_stats && lane == 0) {                       \
    const uint64_t t_ = (uint64_t)clock64();                       \
    ph[k] += t_ - ph_t;                                            \
    ph_t = t_;                                                     \
  }

  const Placement pl = place_units(a, tid, sPlace);
  const int U = a.units_per_head;
  const int grp = pl.grp, n_grp = pl.n_grp, li = pl.li, W = pl.W;
  const bool grouped = pl.grouped, xl = pl.xl;
  const int BH = a.total_units / U;
  const int hg = (BH - grp + n_grp - 1) / n_grp;  // heads of this group
  const int n_units = hg * U;                      // units of this group
  const int stride_static = grouped ? (W / U) * U : a.p_eff;
  uint32_t* work_counter = grouped ? &a.header[20 + grp] : &a.header[1];
  int unit = (a.dynamic == 0 && li >= stride_static) ? n_units : li;

  while (unit < n_units) {
    // head-major: a head's units in a row; unit-major (dynamic schedules
    // only): unit lu of every head of the group in turn
    const int hq = a.unit_major ? unit % hg : unit / U;
    const int lu = a.unit_major ? unit / hg : unit - hq * U;
    const int head = grp + n_grp * hq;
    const size_t hoff = (size_t)head * N * D;
    const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
    const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
    const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
    const T* dOg = reinterpret_cast<const T*>(a.dout) + hoff;
    const float* lse_g = a.lse + (size_t)head * N;
    const float* del_g = a.delta + (size_t)head * N;
    float* dqa = a.dq_accum + hoff;
    T* dqo = reinterpret_cast<T*>(a.dq) + hoff;
    uint32_t* cnt_h = a.counters + (size_t)head * n_sub * NW;
    const int it0 = a.unit_off[lu];
    const int n_items = a.unit_off[lu + 1] - it0;  // <= kMaxUnitItems (checked by the host)
    const int n_steps = n_items * RHO;

    // The unit's work list into LDS.  Every wave has finished the previous
    // unit (including all LDS reads) once it passes this barrier.
    // every wave has finished the previous unit (its last reads of the work
    // list included) before the list is overwritten
    __syncthreads();
    for (int i = tid; i < n_items; i += NT) sItems[i] = a.items[it0 + i];
    __syncthreads();

    frag Kreg[DK], Vreg[DK];
    frag KT[CPW][KK];
    f32x16 accdK[NTD], accdV[NTD];
    int cur_kv = -1;

    // deferred ordered add: partial of the previous sub-tile, held row-major
    // in this wave's LDS area (sRow) from the end of its sub-tile
    f32x4 lv[QT][4];                             // accumulator values read back
    int p_qtile = -1, p_rank = 0, p_flags = 0;  // flags: bit0 last
    bool rel_pending = false;                    // stores issued, counter not yet advanced
    int rel_qtile = 0, rel_rank = 0;

    u32x4 pq[CPT], pdo[CPT];
    float pstat = 0.f;
    // Every sub-tile issues the same vector-memory sequence (accumulator
    // loads, stores, counter peek, prefetch), with unneeded loads sent out of
    // range (they read nothing) or to a valid duplicate: completions are
    // counted in issue order, and a fixed sequence lets each wait cover only
    // the loads it needs instead of everything in flight.
    auto fetch = [&](int g) {
      g = g < n_steps ? g : n_steps - 1;  // past the end: a harmless re-read
      const int qtile = (sItems[g / RHO].x >> 16) * RHO + (g % RHO);
      const int q0 = qtile * BR;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        const int row = c / (D / VEC);
        const int col = (c % (D / VEC)) * VEC;
        const uint32_t off = (uint32_t)((q0 + row) * D + col);
        pq[i] = *reinterpret_cast<const u32x4*>(Qg + off);
        pdo[i] = *reinterpret_cast<const u32x4*>(dOg + off);
      }
      // one load into one register for every lane (lanes past 2*BR re-read a
      // valid element and discard it)
      const float* src = tid < BR ? lse_g + (q0 + tid)
                                  : del_g + (q0 + (tid < 2 * BR ? tid - BR : 0));
      pstat = *src;
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        const int row = c / (D / VEC);
        const int col = (c % (D / VEC)) * VEC;
        *reinterpret_cast<u32x4*>(&sQ[buf][qix(row, col)]) = pq[i];
        *reinterpret_cast<u32x4*>(&sdO[buf][qix(row, col)]) = pdo[i];
      }
      if (tid < BR) sLSE[buf][tid] = pstat * kLog2e;
      else if (tid < 2 * BR) sDel[buf][tid - BR] = pstat;
    };

    auto flush_dkdv = [&]() {
      T* dKg = reinterpret_cast<T*>(a.dk) + hoff;
      T* dVg = reinterpret_cast<T*>(a.dv) + hoff;
#pragma unroll
      for (int nt = 0; nt < NTD; ++nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = (uint32_t)((cur_kv * BC + 32 * w + crow(r, hh)) * D + nt * 32 + l32);
          dKg[off] = E::from_f32(accdK[nt][r] * a.scale);
          dVg[off] = E::from_f32(accdV[nt][r]);
        }
      }
    };

    // this wave's counter for a Q sub-tile
    auto counter = [&](int qtile) { return cnt_h + (size_t)qtile * NW + w; };
    // dQ partials are computed transposed (dQ^T = K^T dS^T): lane <-> Q row,
    // register r <-> column nt*32 + crow(r, h), so registers 4g..4g+3 hold 4
    // consecutive columns and the accumulator moves in 16-byte pieces.
    const __amdgpu_buffer_rsrc_t dq_rs = make_rsrc(dqa, (uint32_t)(N * D * 4));
    // (The atomic schedule keeps dQ untransposed, lane <-> column, so each
    // atomic instruction covers whole rows.)
    // row-major chunk k (0..3) of output tile i for this lane: 4 consecutive
    // columns of one row; 8 lanes cover a 32-column (128-byte) row
    auto chunk_off = [&](int q0, int i, int k) {
      const int nt = col0 + (i / RPW) * NW;
      const int mt = row0 + (i % RPW) * WPC;
      return (uint32_t)((q0 + mt * 32 + (lane >> 3) + 8 * k) * D + nt * 32 + 4 * (lane & 7));
    };
    auto dq_off = [&](int q0, int i, int r) {
      const int nt = col0 + (i / RPW) * NW;
      const int mt = row0 + (i % RPW) * WPC;
      if constexpr (ORDERED) return (uint32_t)((q0 + mt * 32 + l32) * D + nt * 32 + crow(r, hh));
      else return (uint32_t)((q0 + mt * 32 + crow(r, hh)) * D + nt * 32 + l32);
    };

    // Ordered add of the deferred partial.  begin_add (top of the next
    // sub-tile) checks once, without waiting, whether it is this wave's turn
    // and if so starts reading the accumulator; finish_add (after the next
    // sub-tile's products) waits for the turn if it had not come yet, reads,
    // adds and writes back (or writes the final dQ if last).
    bool p_loaded = false;
    auto wait_turn = [&]() {
      const int rank = p_rank;
      if (lane == 0) {
        const uint64_t t0 = (DEBUG && a.wait_stats) ? (uint64_t)clock64() : 0;
        if (DEBUG && a.jitter_seed != 0u) {
          const uint32_t nap =
              hash32(a.jitter_seed ^ (uint32_t)(head * 7919 + p_qtile * 131 + cur_kv * 17 + w)) & 31u;
          for (uint32_t i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(8);
        }
        const bool poisoned = DEBUG && a.poison_q >= 0 && head == 0 && p_qtile == a.poison_q && rank == 0;
        uint32_t polls = 0;
        if (poisoned) polls = wait_counter(counter(p_qtile), 0xFFFFFFFFu, status, spin_limit);
        else if (rank > 0) polls = wait_counter(counter(p_qtile), (uint32_t)rank, status, spin_limit);
        if (DEBUG && a.wait_stats) {
          st_wait += (uint64_t)clock64() - t0;
          st_spun += polls > 0 ? 1u : 0u;
        }
      }
      __builtin_amdgcn_wave_barrier();
    };
    // loads of the accumulator values this wave adds to; `live` false sends
    // them out of the buffer's range (they return 0 and touch no memory)
    auto load_acc = [&](bool live) {
      const int q0 = p_qtile * BR;
      // L2-coherent loads may hit this CU's L1: drop every line read before
      // other workgroups updated it, right before the reads (an add can run
      // after the next KV tile has started, and a unit may visit a Q
      // sub-tile again under a later KV tile)
      if (xl && live) l1_invalidate();
#pragma unroll
      for (int i = 0; i < QT; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t off = live ? 4 * chunk_off(q0, i, k) : kOutOfRange;
          lv[i][k] = xl ? coherent_load4<kXcdCoherent>(dq_rs, off)
                        : coherent_load4<kCoherent>(dq_rs, off);
        }
      p_loaded = live;
    };
    // p_seen: the counter value lane 0 read (without waiting) right after the
    // partial was computed; if it already shows this wave's turn, the
    // accumulator loads start at the top of the next sub-tile.
    uint32_t p_seen = 0;
    auto peek_turn = [&]() { p_seen = load_relaxed_agent(counter(p_qtile)); };
    auto begin_add = [&]() {
      bool ready = p_qtile >= 0 && p_rank > 0 &&
                   __builtin_amdgcn_readfirstlane(p_seen) == (uint32_t)p_rank;
      if (DEBUG && (a.jitter_seed != 0u || a.poison_q >= 0)) ready = false;
      load_acc(ready);
    };
    auto finish_add = [&]() {
      if (DEBUG && a.wait_stats && lane == 0) st_waits += p_rank > 0 ? 1u : 0u;
      if (!p_loaded) {
        wait_turn();
        if (p_rank > 0) load_acc(true);
      }
      const bool last = (p_flags & 1) != 0;
      const int q0 = p_qtile * BR;
      // the partial was written by this wave at the end of the previous
      // sub-tile (one wave's LDS accesses complete in issue order)
      const float* row = sRow[w];
#pragma unroll
      for (int i = 0; i < QT; ++i) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 v = *reinterpret_cast<const f32x4*>(
              &row[rix(i * 32 + (lane >> 3) + 8 * gq, 4 * (lane & 7))]);
          if (p_rank > 0) v = lv[i][gq] + v;
          const uint32_t off = chunk_off(q0, i, gq);
          if (last) {
            v *= a.scale;
            if constexpr (KPL == 8) {
              *reinterpret_cast<uint2*>(&dqo[off]) =
                  make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
            } else {
              *reinterpret_cast<f32x4*>(&dqo[off]) = v;
            }
          } else {
            if (xl) coherent_store4<kXcdCoherent>(dq_rs, 4 * off, v);
            else coherent_store4<kCoherent>(dq_rs, 4 * off, v);
          }
        }
      }
      if (!last) {
        rel_pending = true;
        rel_qtile = p_qtile;
        rel_rank = p_rank;
      }
      p_qtile = -1;
    };
    // Advance the counter of the last ordered add once its stores completed.
    auto release = [&]() {
      if (rel_pending) {
        wait_vm_stores();
        if (lane == 0) advance_counter(counter(rel_qtile), (uint32_t)rel_rank + 1u);
        rel_pending = false;
      }
    };

    if (n_steps > 0) {
      fetch(0);
      stage(0);  // made visible by the barrier of the first KV tile below
    }
    if (n_steps > 1) fetch(1);

    for (int g = 0; g < n_steps; ++g) {
      const int b = g & 1;
      const int2 itm = sItems[g / RHO];
      const int kv = itm.x & 0xFFFF;
      const int qblk = itm.x >> 16;
      const int rank = itm.y & 0xFFFF;
      const int flags = (itm.y >> 30) & 1;
      const int rsub = g % RHO;
      const int qtile = qblk * RHO + rsub;
      const int q0 = qtile * BR;

      if (kv != cur_kv) {
        if (cur_kv >= 0) flush_dkdv();
        cur_kv = kv;
        const int kv0 = kv * BC;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const uint32_t off = (uint32_t)((kv0 + 32 * w + l32) * D + ks * KSTEP + hh * KPL);
          Kreg[ks] = load_frag(Kg + off);
          Vreg[ks] = load_frag(Vg + off);
        }
        // K tile row-major into LDS, then K^T fragments (d on lanes) for dQ.
        // sK's previous readers finished before several barriers since.
        if constexpr (KPL == 8 && D == 64) {
          // bf16: each lane's K fragments are 16-byte row chunks already
          // (row 32w + l32, columns 16ks + 8h ..): write them out, no second
          // read of K
#pragma unroll
          for (int ks = 0; ks < DK; ++ks)
            *reinterpret_cast<uint4*>(&sK[qix(32 * w + l32, ks * KSTEP + hh * KPL)]) =
                __builtin_bit_cast(uint4, Kreg[ks]);
        } else {
          for (int c = tid; c < BC * D / VEC; c += NT) {
            const int row = c / (D / VEC);
            const int col = (c % (D / VEC)) * VEC;
            *reinterpret_cast<uint4*>(&sK[qix(row, col)]) =
                *reinterpret_cast<const uint4*>(Kg + (uint32_t)((kv0 + row) * D + col));
          }
        }
        __syncthreads();
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
          const int nt = col0 + cc * NW;
#pragma unroll
          for (int ks = 0; ks < KK; ++ks) {
            if constexpr (KPL == 8) {
              KT[cc][ks] = tr_frag(sK, qix, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, nt * 32 + gcol, j16);
            } else {
              KT[cc][ks] = load_frag(&sK[(ks * 2 + hh) * LQ + nt * 32 + l32]);
            }
          }
        }
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
          accdK[nt] = zero16();
          accdV[nt] = zero16();
        }
      }


      PHASE(0);  // item decode, KV tile change
      const T* cQ = sQ[b];
      const T* cdO = sdO[b];
      // S = Q K^T and dP = dO V^T for this wave's 32 KV columns
      f32x16 accS[MT], accP[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        accS[mt] = zero16();
        accP[mt] = zero16();
      }
      // in two halves over d: all A fragments of a half are read first, then
      // its MFMAs, so the LDS reads overlap each other and the MFMAs instead
      // of each MFMA waiting on its own operand (the scheduling barriers keep
      // the compiler from interleaving them back)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        frag qa[DK / 2][MT], oa[DK / 2][MT];
#pragma unroll
        for (int k2 = 0; k2 < DK / 2; ++k2)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int off = qix(mt * 32 + l32, (h2 * DK / 2 + k2) * KSTEP + hh * KPL);
            qa[k2][mt] = load_frag(&cQ[off]);
            oa[k2][mt] = load_frag(&cdO[off]);
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k2 = 0; k2 < DK / 2; ++k2)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            accS[mt] = E::mma(qa[k2][mt], Kreg[h2 * DK / 2 + k2], accS[mt]);
            accP[mt] = E::mma(oa[k2][mt], Vreg[h2 * DK / 2 + k2], accP[mt]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }

      // Start reading the accumulator for the previous sub-tile's partial if
      // its turn had already come.  Reading the counter peek waits for every
      // load issued before it (the prefetch too), so it sits behind the S/dP
      // products rather than at the top of the sub-tile.
      PHASE(1);  // S and dP products
      if constexpr (ORDERED) begin_add();
      PHASE(2);  // counter check, accumulator reads issued

      // P and dS; dS^T to LDS.  bf16: P and dS are packed once (hardware
      // RNE conversion) and the packed words serve both the LDS write and the
      // MFMA A operands.  fp32: P and dS stay in place (accS <- P, accP <- dS).
      // pairs flagged partial hide the elements outside lo <= i - j <= hi
      // (the causal diagonal, window edges); uniform across the workgroup
      const bool emask = MASKED && ((itm.y >> 29) & 1);
      const int kvl = 32 * w + l32;
      const int mbase = (qblk - kv) * BC + rsub * BR - kvl;  // i - j = mbase + row
      T* cdSt = sdSt[b];
      uint32_t pw[MT][8], dw[MT][8];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int qb = mt * 32 + 8 * gq + 4 * hh;  // 4 consecutive Q rows
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sLSE[b][qb]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDel[b][qb]);
          float p[4], ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[e] = __builtin_amdgcn_exp2f(accS[mt][4 * gq + e] * a.scale_log2 - l4[e]);
          if (emask) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int dd = mbase + qb + e;
              if (dd < a.mask_lo || dd > a.mask_hi) p[e] = 0.f;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[e] = p[e] * (accP[mt][4 * gq + e] - d4[e]);
          if constexpr (KPL == 8) {
            pw[mt][2 * gq] = pack2_bf16(p[0], p[1]);
            pw[mt][2 * gq + 1] = pack2_bf16(p[2], p[3]);
            dw[mt][2 * gq] = pack2_bf16(ds[0], ds[1]);
            dw[mt][2 * gq + 1] = pack2_bf16(ds[2], ds[3]);
            *reinterpret_cast<uint2*>(&cdSt[kvl * LS + qb]) =
                make_uint2(dw[mt][2 * gq], dw[mt][2 * gq + 1]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              accS[mt][4 * gq + e] = p[e];
              accP[mt][4 * gq + e] = ds[e];
            }
            *reinterpret_cast<f32x4*>(&cdSt[kvl * LS + qb]) = f32x4{ds[0], ds[1], ds[2], ds[3]};
          }
        }
      }

      PHASE(3);  // softmax, dS
      // dV += P^T dO ; dK += dS^T Q   (contraction over this sub-tile's Q rows)
#pragma unroll
      for (int c = 0; c < BR / KSTEP; ++c) {
        constexpr int CPM = 32 / KSTEP;  // chunks per 32-row tile
        const int mt = c / CPM;
        const int cc = c % CPM;
        frag pa, da;
        if constexpr (KPL == 8) {
          pa = __builtin_bit_cast(bf16x8, make_uint4(pw[mt][4 * cc], pw[mt][4 * cc + 1],
                                                     pw[mt][4 * cc + 2], pw[mt][4 * cc + 3]));
          da = __builtin_bit_cast(bf16x8, make_uint4(dw[mt][4 * cc], dw[mt][4 * cc + 1],
                                                     dw[mt][4 * cc + 2], dw[mt][4 * cc + 3]));
        } else {
          pa = accS[mt][cc];
          da = accP[mt][cc];
        }
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
          frag bo, bq;
          if constexpr (KPL == 8) {
            // K slots: Q rows r0+{0..3}, r0+8+{0..3}, r0 = mt*32 + 16cc + 4h
            const int r0 = mt * 32 + 16 * cc + 4 * hh;
            bo = tr_frag(cdO, qix, r0, r0 + 8, nt * 32 + gcol, j16);
            bq = tr_frag(cQ, qix, r0, r0 + 8, nt * 32 + gcol, j16);
          } else {
            const int qrow = mt * 32 + crow(cc, hh);
            bo = load_frag(&cdO[qrow * LQ + nt * 32 + l32]);
            bq = load_frag(&cQ[qrow * LQ + nt * 32 + l32]);
          }
          accdV[nt] = E::mma(pa, bo, accdV[nt]);
          accdK[nt] = E::mma(da, bq, accdK[nt]);
        }
      }

      // stage the next sub-tile into the other buffer (its previous readers,
      // sub-tile g-1, finished before the last barrier)
      PHASE(4);  // dV and dK products
      if (g + 1 < n_steps) stage(b ^ 1);
      PHASE(5);  // staging the next sub-tile
      // finish the previous sub-tile's ordered add behind this one's products
      if constexpr (ORDERED) {
        if (p_qtile >= 0) finish_add();
      }
      PHASE(6);  // previous partial's add
      __syncthreads();  // dS^T of this sub-tile and the next staged sub-tile are complete
      PHASE(7);  // barrier

      // dQ_part = dS K for this wave's output tiles
      f32x16 accQ[QT];
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        const int cc = i / RPW;
        const int mt = row0 + (i % RPW) * WPC;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < KK; ++ks) {
          frag fa;
          if constexpr (KPL == 8) {
            fa = tr_frag(cdSt, six, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, mt * 32 + gcol, j16);
          } else {
            fa = load_frag(&cdSt[(ks * 2 + hh) * LS + mt * 32 + l32]);
          }
          if constexpr (ORDERED) acc = E::mma(KT[cc][ks], fa, acc);  // dQ^T tile
          else acc = E::mma(fa, KT[cc][ks], acc);                    // dQ tile
        }
        accQ[i] = acc;
      }
      // the previous partial's stores (issued before the barrier) complete
      // here; advance its counter before issuing the next prefetch, so the
      // wait does not include loads that were just issued
      PHASE(8);  // dQ product
      if constexpr (ORDERED) release();
      PHASE(9);  // hand-off
      fetch(g + 2);

      if (DEBUG && a.partials != nullptr) {
        float* pp = a.partials + (((size_t)head * a.n_tiles + kv) * N) * D;
#pragma unroll
        for (int i = 0; i < QT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) pp[dq_off(q0, i, r)] = accQ[i][r];
      }

      if constexpr (ORDERED) {
        // transpose the partial to row-major through this wave's LDS area
        // now; its ordered add is finished during the next sub-tile
        float* row = sRow[w];
#pragma unroll
        for (int i = 0; i < QT; ++i)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<f32x4*>(&row[rix(i * 32 + l32, 8 * gq + 4 * hh)]) =
                f32x4{accQ[i][4 * gq], accQ[i][4 * gq + 1], accQ[i][4 * gq + 2],
                      accQ[i][4 * gq + 3]};
        p_qtile = qtile;
        p_rank = rank;
        p_flags = flags;
        peek_turn();
      } else {
#pragma unroll
        for (int i = 0; i < QT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) atomic_add_f32(&dqa[dq_off(q0, i, r)], accQ[i][r]);
      }
      PHASE(10);  // prefetch, partial staging, counter read (or atomic adds)
    }
    if (cur_kv >= 0) flush_dkdv();
    if constexpr (ORDERED) {
      release();
      if (p_qtile >= 0) {
        begin_add();
        finish_add();
      }
      release();
    }

    // next unit
    if (a.dynamic) {
      if (tid == 0)
        sUnit = (int)__hip_atomic_fetch_add(work_counter, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + W;
      __syncthreads();
      unit = sUnit;
      __syncthreads();
    } else {
      unit += stride_static;
    }
  }
  if (DEBUG && a.wait_stats != nullptr && lane == 0) {
    uint64_t* st = a.wait_stats + ((size_t)blockIdx.x * NW + w) * 4;
    st[0] = st_wait;
    st[1] = st_waits;
    st[2] = st_spun;
    st[3] = (uint64_t)clock64() - st_t0;
  }
  if (DEBUG && a.phase_stats != nullptr && lane == 0) {
    uint64_t* st = a.phase_stats + ((size_t)blockIdx.x * NW + w) * 16;
    for (int k = 0; k < kPhases; ++k) st[k] = ph[k];
    st[15] = (uint64_t)clock64() - ph_t0;
  }
#undef PHASE
}

// ------------------------------------------------------------ dispatch

// DEBUG instantiations carry the test hooks (jitter, poison, partials dump,
// wait statistics); the production kernels have none of their code.
template <typename T, int D, int BC, int BR, bool DEBUG>
static void* pick2(bool masked, bool ordered) {
  if (masked)
    return ordered ? (void*)bwd_kernel<T, D, BC, BR, true, true, DEBUG>
                   : (void*)bwd_kernel<T, D, BC, BR, true, false, DEBUG>;
  return ordered ? (void*)bwd_kernel<T, D, BC, BR, false, true, DEBUG>
                 : (void*)bwd_kernel<T, D, BC, BR, false, false, DEBUG>;
}

template <typename T, int D, int BC, int BR>
static void* pick(bool masked, bool ordered, bool debug) {
  return debug ? pick2<T, D, BC, BR, true>(masked, ordered)
               : pick2<T, D, BC, BR, false>(masked, ordered);
}

static void* select_bwd(int dtype, int d, bool masked, bool ordered, bool debug, int* threads) {
  if (dtype == 1 && d == 128) { *threads = 256; return pick<bf16_t, 128, 128, 32>(masked, ordered, debug); }
  if (dtype == 1 && d == 64) { *threads = 256; return pick<bf16_t, 64, 128, 64>(masked, ordered, debug); }
  if (dtype == 0 && d == 64) { *threads = 128; return pick<float, 64, 64, 64>(masked, ordered, debug); }
  if (dtype == 0 && d == 128) { *threads = 128; return pick<float, 128, 64, 32>(masked, ordered, debug); }
  return nullptr;
}

void bwd_tiles(int dtype, int d, int* bc, int* br) {
  if (dtype == 1) { *bc = 128; *br = (d == 128) ? 32 : 64; }
  else { *bc = 64; *br = (d == 128) ? 32 : 64; }
}

int bwd_waves(int dtype, int d) {
  int bc = 0, br = 0;
  bwd_tiles(dtype, d, &bc, &br);
  return bc / 32;
}

hipError_t bwd_max_coresident(int dtype, int d, bool masked, bool ordered, int* blocks) {
  int threads = 0;
  int per_cu = 0;
  // the test-hook instantiations must fit as many workgroups as production
  for (int dbg = 0; dbg < 2; ++dbg) {
    void* f = select_bwd(dtype, d, masked, ordered, dbg != 0, &threads);
    if (!f) return hipErrorInvalidValue;
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, threads, 0);
    if (e != hipSuccess) return e;
    per_cu = dbg == 0 ? n : (n < per_cu ? n : per_cu);
  }
  hipError_t e = hipSuccess;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_bwd(int dtype, int d, bool masked, bool ordered, const BwdArgs& a, int grid,
                      hipStream_t stream) {
  int threads = 0;
  const bool debug = a.jitter_seed != 0u || a.poison_q >= 0 || a.partials != nullptr ||
                     a.wait_stats != nullptr || a.phase_stats != nullptr;
  void* f = select_bwd(dtype, d, masked, ordered, debug, &threads);
  if (!f) return hipErrorInvalidValue;
  BwdArgs copy = a;
  void* args[] = {&copy};
  // Cooperative launch: the runtime refuses a grid whose workgroups cannot
  // all be resident, which the ordered waits rely on.
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(threads), args, 0, stream);
}

}  // namespace dash
