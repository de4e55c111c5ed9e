// Deterministic attention backward, wave-pair layout (bf16, d = 128).
//
// The same method, schedules, tables and ordered dQ hand-off as the
// one-wave-per-slice kernel (attn_bwd.hip), with each 32-row KV slice of a
// workgroup's KV tile split between two waves, so that two waves share each
// SIMD at no more than 256 registers: while one waits for memory the other
// can issue MFMAs.  Results are bit-identical to the other layout: every
// product, exponential and add is computed in the same order.
#include "common.hpp"
#include "launch.hpp"
#include "placement.hpp"

namespace dash {

// bf16, d = 128, BC = 128, BR = 32, 8 waves (two per SIMD, at most 256
// registers each).  Wave s (0..3) = "A" of KV slice s: K and K^T fragments,
// S, P, dV and the dQ product.  Wave s + 4 = "B" of slice s: V fragments,
// dP, dS, dK and the ordered add's memory work.  P passes from A to B, the
// dQ partial from A to B, through LDS.
template <bool MASKED, bool ORDERED, bool DEBUG>
__global__ void __launch_bounds__(512, 1) bwd_pair_kernel(BwdArgs a) {
  using T = bf16_t;
  using E = Elt<T>;
  using frag = typename E::frag;
  constexpr int D = 128, BC = 128, BR = 32;
  constexpr int NW = 4;               // KV slices (= ordered-add waves, counter layout)
  constexpr int NT = 512;
  constexpr int RHO = BC / BR;
  constexpr int KPL = 8, KSTEP = 16, VEC = 8;
  constexpr int DK = D / KSTEP;       // 8
  constexpr int KK = BC / KSTEP;      // 8
  constexpr int NTD = D / 32;         // 4
  constexpr int LQ = D;
  constexpr int LS = BR + 4;
  constexpr int CPT = BR * D / VEC / NT;  // 1
  static_assert(CPT * VEC * NT == BR * D, "sub-tile load must split evenly");

  __shared__ __align__(16) T sQ[2][BR * LQ];
  __shared__ __align__(16) T sdO[2][BR * LQ];
  __shared__ __align__(16) T sdSt[2][BC * LS];
  __shared__ __align__(16) T sK[BC * LQ];
  __shared__ __align__(16) float sP[NW][64 * 16];     // fp32 P of each slice, per lane its 16 values
  __shared__ __align__(16) float sLSE[2][BR];
  __shared__ __align__(16) float sDel[2][BR];
  __shared__ int2 sItems[kMaxUnitItems];
  constexpr int LR = 32;
  __shared__ __align__(16) float sRow[ORDERED ? NW : 1][ORDERED ? 32 * LR : 4];
  __shared__ int sUnit;
  __shared__ int sPlace[5];
  const auto qix = [](int r, int c) { return r * LQ + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7); };
  const auto six = [](int r, int c) { return r * LS + c; };
  const auto rix = [](int r, int c) { return r * LR + (((c >> 2) ^ ((r >> 1) & 7)) << 2) + (c & 3); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;             // 0..7
  const bool isA = wv < NW;
  const int w = wv & 3;                // KV slice
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int j16 = lane & 15;
  const int gcol = 16 * ((lane >> 4) & 1);
  const int N = a.N;
  const int n_sub = N / BR;
  uint32_t* status = a.header;
  const uint32_t spin_limit = a.spin_limit;
  const int col0 = w;

  uint64_t st_wait = 0, st_waits = 0, st_spun = 0;
  const uint64_t st_t0 = (DEBUG && a.wait_stats) ? (uint64_t)clock64() : 0;
  // phase timer (test hook): lane 0 of each wave adds the shader-clock
  // cycles since the previous mark to the phase that just ended; the
  // phases of A waves: 0 item decode and KV tile changes, 1 S products,
  // 2 softmax and P to LDS, 3 the P barrier, 4 dV products, 5 staging,
  // 6 the sub-tile barrier, 7 dQ product and partial to LDS, 8 prefetch;
  // of B waves: 0, 1 dP products and counter check, 2 -, 3 the P barrier,
  // 4 dS and dK products, 5 staging, 6 the ordered add and the sub-tile
  // barrier, 7 the hand-off, 8 prefetch and counter read
  uint64_t ph[9] = {};
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
  const int hg = (BH - grp + n_grp - 1) / n_grp;
  const int n_units = hg * U;
  const int stride_static = grouped ? (W / U) * U : a.p_eff;
  uint32_t* work_counter = grouped ? &a.header[20 + grp] : &a.header[1];
  const int unit0 = (a.dynamic == 0 && li >= stride_static) ? n_units : li;
  // one copy of the unit loop per role, so that each role's registers are
  // allocated for its own values only (both copies pass the same barriers
  // in the same order)
  auto run = [&](auto role) {
    constexpr bool IS_A = decltype(role)::value;
    int unit = unit0;
    while (unit < n_units) {
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
      const int n_items = a.unit_off[lu + 1] - it0;
      const int n_steps = n_items * RHO;

      __syncthreads();
      for (int i = tid; i < n_items; i += NT) sItems[i] = a.items[it0 + i];
      __syncthreads();

      frag KV[DK];        // A: K fragments; B: V fragments
      frag KT[KK];        // A: K^T fragments (d on lanes) for dQ
      f32x16 acc[NTD];    // A: dV; B: dK
      int cur_kv = -1;

      f32x4 lv[4];
      int p_qtile = -1, p_rank = 0, p_flags = 0;
      bool rel_pending = false;
      int rel_qtile = 0, rel_rank = 0;

      u32x4 pq[CPT], pdo[CPT];
      float pstat = 0.f;
      auto fetch = [&](int g) {
        g = g < n_steps ? g : n_steps - 1;
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
      auto flush = [&]() {
        T* dst = reinterpret_cast<T*>(IS_A ? a.dv : a.dk) + hoff;
        const float sc = IS_A ? 1.f : a.scale;
  #pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t off = (uint32_t)((cur_kv * BC + 32 * w + crow(r, hh)) * D + nt * 32 + l32);
            dst[off] = E::from_f32(acc[nt][r] * sc);
          }
        }
      };

      auto counter = [&](int qtile) { return cnt_h + (size_t)qtile * NW + w; };
      const __amdgpu_buffer_rsrc_t dq_rs = make_rsrc(dqa, (uint32_t)(N * D * 4));
      auto chunk_off = [&](int q0, int k) {
        return (uint32_t)((q0 + (lane >> 3) + 8 * k) * D + col0 * 32 + 4 * (lane & 7));
      };
      auto dq_off = [&](int q0, int r) {
        if constexpr (ORDERED) return (uint32_t)((q0 + l32) * D + col0 * 32 + crow(r, hh));
        else return (uint32_t)((q0 + crow(r, hh)) * D + col0 * 32 + l32);
      };

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
      auto load_acc = [&](bool live) {
        const int q0 = p_qtile * BR;
        if (xl && live) l1_invalidate();
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t off = live ? 4 * chunk_off(q0, k) : kOutOfRange;
          lv[k] = xl ? coherent_load4<kXcdCoherent>(dq_rs, off) : coherent_load4<kCoherent>(dq_rs, off);
        }
        p_loaded = live;
      };
      uint32_t p_seen = 0;
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
        const float* row = sRow[w];
  #pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 v = *reinterpret_cast<const f32x4*>(&row[rix((lane >> 3) + 8 * gq, 4 * (lane & 7))]);
          if (p_rank > 0) v = lv[gq] + v;
          const uint32_t off = chunk_off(q0, gq);
          if (last) {
            v *= a.scale;
            *reinterpret_cast<uint2*>(&dqo[off]) =
                make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
          } else {
            if (xl) coherent_store4<kXcdCoherent>(dq_rs, 4 * off, v);
            else coherent_store4<kCoherent>(dq_rs, 4 * off, v);
          }
        }
        if (!last) {
          rel_pending = true;
          rel_qtile = p_qtile;
          rel_rank = p_rank;
        }
        p_qtile = -1;
      };
      auto release = [&]() {
        if (rel_pending) {
          wait_vm_stores();
          if (lane == 0) advance_counter(counter(rel_qtile), (uint32_t)rel_rank + 1u);
          rel_pending = false;
        }
      };

      if (n_steps > 0) {
        fetch(0);
        stage(0);
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
          if (cur_kv >= 0) flush();
          cur_kv = kv;
          const int kv0 = kv * BC;
          const T* src = IS_A ? Kg : Vg;
  #pragma unroll
          for (int ks = 0; ks < DK; ++ks) {
            const uint32_t off = (uint32_t)((kv0 + 32 * w + l32) * D + ks * KSTEP + hh * KPL);
            KV[ks] = load_frag(src + off);
          }
          for (int c = tid; c < BC * D / VEC; c += NT) {
            const int row = c / (D / VEC);
            const int col = (c % (D / VEC)) * VEC;
            *reinterpret_cast<uint4*>(&sK[qix(row, col)]) =
                *reinterpret_cast<const uint4*>(Kg + (uint32_t)((kv0 + row) * D + col));
          }
          __syncthreads();
          if constexpr (IS_A) {
  #pragma unroll
            for (int ks = 0; ks < KK; ++ks)
              KT[ks] = tr_frag(sK, qix, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, col0 * 32 + gcol, j16);
          }
  #pragma unroll
          for (int nt = 0; nt < NTD; ++nt) acc[nt] = zero16();
        }

        PHASE(0);
        const T* cQ = sQ[b];
        const T* cdO = sdO[b];
        // A: S = Q K^T; B: dP = dO V^T (this slice's 32 KV columns)
        f32x16 accX = zero16();
        {
          const T* src = IS_A ? cQ : cdO;
  #pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            frag xa[DK / 2];
  #pragma unroll
            for (int k2 = 0; k2 < DK / 2; ++k2)
              xa[k2] = load_frag(&src[qix(l32, (h2 * DK / 2 + k2) * KSTEP + hh * KPL)]);
            __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
            for (int k2 = 0; k2 < DK / 2; ++k2) accX = E::mma(xa[k2], KV[h2 * DK / 2 + k2], accX);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const int kvl = 32 * w + l32;
        uint32_t pw[8];
        if constexpr (!IS_A && ORDERED) begin_add();
        PHASE(1);
        if constexpr (IS_A) {

          const bool emask = MASKED && ((itm.y >> 29) & 1);
          const int mbase = (qblk - kv) * BC + rsub * BR - kvl;
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int qb = 8 * gq + 4 * hh;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sLSE[b][qb]);
            float p[4];
  #pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(accX[4 * gq + e] * a.scale_log2 - l4[e]);
            if (emask) {
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int dd = mbase + qb + e;
                if (dd < a.mask_lo || dd > a.mask_hi) p[e] = 0.f;
              }
            }
            pw[2 * gq] = pack2_bf16(p[0], p[1]);
            pw[2 * gq + 1] = pack2_bf16(p[2], p[3]);
            *reinterpret_cast<f32x4*>(&sP[w][lane * 16 + 4 * gq]) = f32x4{p[0], p[1], p[2], p[3]};
          }
        }
        PHASE(2);
        __syncthreads();  // P of every slice visible to its B wave
        PHASE(3);
        if constexpr (IS_A) {
          // dV += P^T dO
  #pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const frag pa = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * cc], pw[4 * cc + 1],
                                                                  pw[4 * cc + 2], pw[4 * cc + 3]));
  #pragma unroll
            for (int nt = 0; nt < NTD; ++nt) {
              const int r0 = 16 * cc + 4 * hh;
              const frag bo = tr_frag(cdO, qix, r0, r0 + 8, nt * 32 + gcol, j16);
              acc[nt] = E::mma(pa, bo, acc[nt]);
            }
          }
        } else {
          // dS = P (dP - delta); dS^T to LDS; dK += dS^T Q
          uint32_t dw[8];
          T* cdSt = sdSt[b];
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int qb = 8 * gq + 4 * hh;
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDel[b][qb]);
            float ds[4];
            const f32x4 pp = *reinterpret_cast<const f32x4*>(&sP[w][lane * 16 + 4 * gq]);
  #pragma unroll
            for (int e = 0; e < 4; ++e) ds[e] = pp[e] * (accX[4 * gq + e] - d4[e]);
            dw[2 * gq] = pack2_bf16(ds[0], ds[1]);
            dw[2 * gq + 1] = pack2_bf16(ds[2], ds[3]);
            *reinterpret_cast<uint2*>(&cdSt[kvl * LS + qb]) = make_uint2(dw[2 * gq], dw[2 * gq + 1]);
          }
  #pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const frag da = __builtin_bit_cast(bf16x8, make_uint4(dw[4 * cc], dw[4 * cc + 1],
                                                                  dw[4 * cc + 2], dw[4 * cc + 3]));
  #pragma unroll
            for (int nt = 0; nt < NTD; ++nt) {
              const int r0 = 16 * cc + 4 * hh;
              const frag bq = tr_frag(cQ, qix, r0, r0 + 8, nt * 32 + gcol, j16);
              acc[nt] = E::mma(da, bq, acc[nt]);
            }
          }
        }

        PHASE(4);
        if (g + 1 < n_steps) stage(b ^ 1);
        PHASE(5);
        if constexpr (ORDERED) {
          if (!IS_A && p_qtile >= 0) finish_add();
        }
        __syncthreads();  // dS^T of this sub-tile and the next staged sub-tile are complete
        PHASE(6);

        if constexpr (IS_A) {
          // dQ_part = dS K (transposed for the ordered add) for column tile w
          f32x16 accQ = zero16();
          const T* cdSt = sdSt[b];
  #pragma unroll
          for (int ks = 0; ks < KK; ++ks) {
            const frag fa = tr_frag(cdSt, six, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, gcol, j16);
            if constexpr (ORDERED) accQ = E::mma(KT[ks], fa, accQ);
            else accQ = E::mma(fa, KT[ks], accQ);
          }
          if (DEBUG && a.partials != nullptr) {
            float* pp = a.partials + (((size_t)head * a.n_tiles + kv) * N) * D;
  #pragma unroll
            for (int r = 0; r < 16; ++r) pp[dq_off(q0, r)] = accQ[r];
          }
          if constexpr (ORDERED) {
            // row-major into this slice's LDS area; its B wave adds it during
            // the next sub-tile (after the next barrier)
            float* row = sRow[w];
  #pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              *reinterpret_cast<f32x4*>(&row[rix(l32, 8 * gq + 4 * hh)]) =
                  f32x4{accQ[4 * gq], accQ[4 * gq + 1], accQ[4 * gq + 2], accQ[4 * gq + 3]};
          } else {
  #pragma unroll
            for (int r = 0; r < 16; ++r) atomic_add_f32(&dqa[dq_off(q0, r)], accQ[r]);
          }
        }
        if constexpr (ORDERED) {
          if constexpr (!IS_A) {
            release();
            p_qtile = qtile;
            p_rank = rank;
            p_flags = flags;
          }
        }
        PHASE(7);
        fetch(g + 2);
        if constexpr (ORDERED) {
          if constexpr (!IS_A) p_seen = load_relaxed_agent(counter(p_qtile));
        }
        PHASE(8);
      }
      if (cur_kv >= 0) flush();
      // the last partial, written by the A waves after the last barrier, is
      // complete before the B waves add it
      __syncthreads();
      if constexpr (ORDERED) {
        if constexpr (!IS_A) {
          release();
          if (p_qtile >= 0) {
            begin_add();
            finish_add();
          }
          release();
        }
      }

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
  };
  if (isA) run(std::true_type{});
  else run(std::false_type{});
  if (DEBUG && a.phase_stats != nullptr && lane == 0) {
    uint64_t* st = a.phase_stats + ((size_t)blockIdx.x * 8 + (isA ? w : 4 + w)) * 16;
    for (int k = 0; k < 9; ++k) st[k] = ph[k];
    st[14] = isA ? 1u : 2u;
    st[15] = (uint64_t)clock64() - ph_t0;
  }
#undef PHASE
  if (DEBUG && a.wait_stats != nullptr && lane == 0 && !isA) {
    uint64_t* st = a.wait_stats + ((size_t)blockIdx.x * NW + w) * 4;
    st[0] = st_wait;
    st[1] = st_waits;
    st[2] = st_spun;
    st[3] = (uint64_t)clock64() - st_t0;
  }
}

template <bool DEBUG>
static void* pick_pair(bool masked, bool ordered) {
  if (masked)
    return ordered ? (void*)bwd_pair_kernel<true, true, DEBUG> : (void*)bwd_pair_kernel<true, false, DEBUG>;
  return ordered ? (void*)bwd_pair_kernel<false, true, DEBUG> : (void*)bwd_pair_kernel<false, false, DEBUG>;
}

hipError_t bwd_pair_max_coresident(bool masked, bool ordered, int* blocks) {
  int per_cu = 0;
  for (int dbg = 0; dbg < 2; ++dbg) {
    void* f = dbg ? pick_pair<true>(masked, ordered) : pick_pair<false>(masked, ordered);
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 512, 0);
    if (e != hipSuccess) return e;
    per_cu = dbg == 0 ? n : (n < per_cu ? n : per_cu);
  }
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_bwd_pair(bool masked, bool ordered, const BwdArgs& a, int grid,
                           hipStream_t stream) {
  const bool debug = a.jitter_seed != 0u || a.poison_q >= 0 || a.partials != nullptr ||
                     a.wait_stats != nullptr || a.phase_stats != nullptr;
  void* f = debug ? pick_pair<true>(masked, ordered) : pick_pair<false>(masked, ordered);
  BwdArgs copy = a;
  void* args[] = {&copy};
  // cooperative: every workgroup resident, which the ordered waits rely on
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(512), args, 0, stream);
}

}  // namespace dash
