// Persistent deterministic attention backward for gfx950.
//
// One workgroup owns one KV tile (BC rows) at a time and keeps that tile's
// dK and dV accumulators in registers for as long as it works on it (the
// DASH explainer, "Technisches Resuemee" 2.1: one KV tile's operations run
// as an uninterrupted chain on one processor with register-resident
// accumulation).  For every Q block in its schedule it recomputes, per Q
// sub-tile of BR rows:
//   S   = Q K^T                (MFMA; K held in registers)
//   P   = exp(s S - LSE)       (exactly 0 where the causal mask hides a key)
//   dP  = dO V^T               (MFMA; V held in registers)
//   dS  = P (dP - delta)
//   dV += P^T dO ; dK += dS^T Q  (MFMA, accumulators in registers)
//   dQ_part = dS K             (MFMA, dS staged through LDS)
// and adds dQ_part into the fp32 accumulator of that Q sub-tile.  With an
// ordered schedule the add waits until the sub-tile's counter equals this
// tile's rank in the dQ order and then advances the counter, so the adds
// happen in one fixed order (explainer section 1: fixed accumulation order
// for dQ); with the atomic schedule the adds are unordered.
//
// The workgroups form a persistent grid: each takes units (work lists from
// the schedule tables) either from a device work counter in increasing
// order (schedules whose waits point only to earlier units) or in
// head-aligned rounds (shift, whose waits point to other units of the same
// head, all of which are then resident).
//
// Operand placement (see common.hpp for the MFMA layouts):
//   S and dP are computed as (Q-rows x KV-cols), so the accumulators hold
//   KV on lanes and Q rows in registers; reused directly as the A operand
//   of dV += P^T dO and dK += dS^T Q, whose B operands (dO, Q with Q rows
//   in the K slots) come from transposed LDS copies sdOt and sQt.
//   dQ = dS K needs dS with Q rows on lanes: dS goes through LDS (sdS),
//   K through a transposed LDS copy sKt written once per KV tile.
#include "common.hpp"
#include "launch.hpp"

namespace dash {

template <typename T, int D, int BC, int BR, bool CAUSAL, bool ORDERED>
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
  constexpr int MT = BR / 32;          // 32-row tiles of a Q sub-tile
  constexpr int NTD = D / 32;          // 32-column tiles over d
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LQ = D + PAD;          // row stride of sQ, sdO  ([q][d])
  constexpr int LQT = BR + PAD;        // row stride of sQt, sdOt ([d][q])
  constexpr int LS = BC + PAD;         // row stride of sdS ([q][kv]) and sKt ([d][kv])
  constexpr int CPT = BR * D / VEC / NT;  // 16-byte chunks per thread per tensor
  constexpr int QTILES = MT * NTD;     // dQ output tiles per sub-tile
  constexpr int TPW = QTILES / NW;     // dQ tiles per wave
  static_assert(BC % BR == 0 && BR % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(QTILES % NW == 0, "dQ tiles must split evenly over waves");
  static_assert(CPT * VEC * NT == BR * D, "sub-tile load must split evenly");
  static_assert(NT >= 2 * BR, "LSE/delta staging needs 2*BR threads");

  __shared__ __align__(16) T sQ[BR * LQ];
  __shared__ __align__(16) T sdO[BR * LQ];
  __shared__ __align__(16) T sQt[D * LQT];
  __shared__ __align__(16) T sdOt[D * LQT];
  __shared__ __align__(16) T sdS[BR * LS];
  __shared__ __align__(16) T sKt[D * LS];
  __shared__ float sLSE[BR];
  __shared__ float sDel[BR];
  __shared__ int sUnit;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int N = a.N;
  const int n_sub = N / BR;
  uint32_t* status = a.header;
  const uint32_t spin_limit = a.spin_limit;

  if (a.dynamic == 0 && (int)blockIdx.x >= a.p_eff) return;
  int unit = blockIdx.x;

  while (unit < a.total_units) {
    const int head = unit / a.units_per_head;
    const int lu = unit - head * a.units_per_head;
    const size_t hoff = (size_t)head * N * D;
    const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
    const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
    const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
    const T* dOg = reinterpret_cast<const T*>(a.dout) + hoff;
    const float* lse_g = a.lse + (size_t)head * N;
    const float* del_g = a.delta + (size_t)head * N;
    const int it0 = a.unit_off[lu];
    const int it1 = a.unit_off[lu + 1];
    const int n_steps = (it1 - it0) * RHO;

    frag Kreg[DK], Vreg[DK];
    f32x16 accdK[NTD], accdV[NTD];
    int cur_kv = -1;

    // prefetch registers for the next Q sub-tile
    uint4 pq[CPT], pdo[CPT];
    float pstat = 0.f;
    auto fetch = [&](int g) {
      const int2 itm = a.items[it0 + g / RHO];
      const int qtile = (itm.x >> 16) * RHO + (g % RHO);
      const int q0 = qtile * BR;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        const int row = c / (D / VEC);
        const int col = (c % (D / VEC)) * VEC;
        pq[i] = *reinterpret_cast<const uint4*>(Qg + (size_t)(q0 + row) * D + col);
        pdo[i] = *reinterpret_cast<const uint4*>(dOg + (size_t)(q0 + row) * D + col);
      }
      if (tid < BR) pstat = lse_g[q0 + tid] * kLog2e;
      else if (tid < 2 * BR) pstat = del_g[q0 + tid - BR];
    };

    auto flush_dkdv = [&]() {
      T* dKg = reinterpret_cast<T*>(a.dk) + hoff;
      T* dVg = reinterpret_cast<T*>(a.dv) + hoff;
#pragma unroll
      for (int nt = 0; nt < NTD; ++nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = cur_kv * BC + 32 * w + crow(r, hh);
          const int col = nt * 32 + l32;
          dKg[(size_t)row * D + col] = E::from_f32(accdK[nt][r] * a.scale);
          dVg[(size_t)row * D + col] = E::from_f32(accdV[nt][r]);
        }
      }
    };

    if (n_steps > 0) fetch(0);

    for (int g = 0; g < n_steps; ++g) {
      const int2 itm = a.items[it0 + g / RHO];
      const int kv = itm.x & 0xFFFF;
      const int qblk = itm.x >> 16;
      const int rank = itm.y;
      const int rsub = g % RHO;
      const int qtile = qblk * RHO + rsub;
      const int q0 = qtile * BR;

      if (kv != cur_kv) {
        if (cur_kv >= 0) flush_dkdv();
        cur_kv = kv;
        const int kv0 = kv * BC;
        // K, V as B operands (KV rows on lanes, d in the K slots)
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const size_t off = (size_t)(kv0 + 32 * w + l32) * D + ks * KSTEP + hh * KPL;
          Kreg[ks] = load_frag(Kg + off);
          Vreg[ks] = load_frag(Vg + off);
        }
        // K^T into LDS for the dQ product (previous readers passed the
        // barrier that ended the last sub-tile)
        for (int c = tid; c < BC * D / VEC; c += NT) {
          const int row = c / (D / VEC);
          const int col = (c % (D / VEC)) * VEC;
          const uint4 raw = *reinterpret_cast<const uint4*>(Kg + (size_t)(kv0 + row) * D + col);
          const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int j = 0; j < VEC; ++j) sKt[(col + j) * LS + row] = e[j];
        }
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
          accdK[nt] = zero16();
          accdV[nt] = zero16();
        }
      }

      // stage the prefetched Q / dO sub-tile (row-major and transposed)
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        const int row = c / (D / VEC);
        const int col = (c % (D / VEC)) * VEC;
        *reinterpret_cast<uint4*>(&sQ[row * LQ + col]) = pq[i];
        *reinterpret_cast<uint4*>(&sdO[row * LQ + col]) = pdo[i];
        const T* eq = reinterpret_cast<const T*>(&pq[i]);
        const T* ed = reinterpret_cast<const T*>(&pdo[i]);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          sQt[(col + j) * LQT + row] = eq[j];
          sdOt[(col + j) * LQT + row] = ed[j];
        }
      }
      if (tid < BR) sLSE[tid] = pstat;
      else if (tid < 2 * BR) sDel[tid - BR] = pstat;
      __syncthreads();

      if (g + 1 < n_steps) fetch(g + 1);

      // S = Q K^T and dP = dO V^T for this wave's 32 KV columns
      f32x16 accS[MT], accP[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        accS[mt] = zero16();
        accP[mt] = zero16();
      }
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int off = (mt * 32 + l32) * LQ + ks * KSTEP + hh * KPL;
          accS[mt] = E::mma(load_frag(&sQ[off]), Kreg[ks], accS[mt]);
          accP[mt] = E::mma(load_frag(&sdO[off]), Vreg[ks], accP[mt]);
        }
      }

      // P and dS, in place (accS <- P, accP <- dS)
      const bool diag = CAUSAL && (qblk == kv);
      const int kvl = 32 * w + l32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = mt * 32 + crow(r, hh);
          float p = __builtin_amdgcn_exp2f(accS[mt][r] * a.scale_log2 - sLSE[ql]);
          if (diag && kvl > rsub * BR + ql) p = 0.f;
          const float ds = p * (accP[mt][r] - sDel[ql]);
          accS[mt][r] = p;
          accP[mt][r] = ds;
          sdS[ql * LS + kvl] = E::from_f32(ds);
        }
      }

      // dV += P^T dO ; dK += dS^T Q   (contraction over this sub-tile's Q rows)
#pragma unroll
      for (int c = 0; c < BR / KSTEP; ++c) {
        constexpr int CPM = 32 / KSTEP;  // chunks per 32-row tile
        const int mt = c / CPM;
        const int cc = c % CPM;
        frag pa, da;
        if constexpr (KPL == 8) {
          float tp[8], td[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            tp[s] = accS[mt][8 * cc + s];
            td[s] = accP[mt][8 * cc + s];
          }
          pa = pack_bf16x8(tp);
          da = pack_bf16x8(td);
        } else {
          pa = accS[mt][cc];
          da = accP[mt][cc];
        }
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
          const int dcol = nt * 32 + l32;
          frag bo, bq;
          if constexpr (KPL == 8) {
            // rows crow(8cc+s, hh): 16cc + 4hh + {0..3} and 16cc + 8 + 4hh + {0..3}
            const int base = dcol * LQT + mt * 32 + 16 * cc + 4 * hh;
            u16x8 uo, uq;
            const u16x4 o0 = *reinterpret_cast<const u16x4*>(&sdOt[base]);
            const u16x4 o1 = *reinterpret_cast<const u16x4*>(&sdOt[base + 8]);
            const u16x4 q0v = *reinterpret_cast<const u16x4*>(&sQt[base]);
            const u16x4 q1v = *reinterpret_cast<const u16x4*>(&sQt[base + 8]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              uo[s] = o0[s];
              uo[s + 4] = o1[s];
              uq[s] = q0v[s];
              uq[s + 4] = q1v[s];
            }
            bo = __builtin_bit_cast(bf16x8, uo);
            bq = __builtin_bit_cast(bf16x8, uq);
          } else {
            const int qrow = mt * 32 + crow(cc, hh);
            bo = load_frag(&sdOt[dcol * LQT + qrow]);
            bq = load_frag(&sQt[dcol * LQT + qrow]);
          }
          accdV[nt] = E::mma(pa, bo, accdV[nt]);
          accdK[nt] = E::mma(da, bq, accdK[nt]);
        }
      }
      __syncthreads();  // sdS complete

      // dQ_part = dS K for this wave's output tiles
      f32x16 accQ[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = w + i * NW;
        const int mt = t / NTD;
        const int nt = t % NTD;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < BC / KSTEP; ++ks) {
          const frag fa = load_frag(&sdS[(mt * 32 + l32) * LS + ks * KSTEP + hh * KPL]);
          const frag fb = load_frag(&sKt[(nt * 32 + l32) * LS + ks * KSTEP + hh * KPL]);
          acc = E::mma(fa, fb, acc);
        }
        accQ[i] = acc;
      }

      // add into the dQ accumulator, in rank order when ORDERED
      uint32_t* cnt = a.counters + (size_t)head * n_sub + qtile;
      if constexpr (ORDERED) {
        if (tid == 0) {
          if (a.jitter_seed != 0u) {
            uint32_t nap = hash32(a.jitter_seed ^ (uint32_t)(head * 7919 + qtile * 131 + kv)) & 31u;
            for (uint32_t i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(8);
          }
          uint32_t target = (uint32_t)rank;
          if (a.poison_q >= 0 && head == 0 && qtile == a.poison_q && rank == 0) target = 0xFFFFFFFFu;
          wait_counter(cnt, target, status, spin_limit);
        }
        __syncthreads();
      }
      float* dqa = a.dq_accum + (size_t)head * N * D;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = w + i * NW;
        const int mt = t / NTD;
        const int nt = t % NTD;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = q0 + mt * 32 + crow(r, hh);
          const int col = nt * 32 + l32;
          atomic_add_f32(&dqa[(size_t)row * D + col], accQ[i][r]);
        }
      }
      if (a.partials != nullptr) {
        float* pp = a.partials + (((size_t)head * a.n_tiles + kv) * N) * D;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int t = w + i * NW;
          const int mt = t / NTD;
          const int nt = t % NTD;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = q0 + mt * 32 + crow(r, hh);
            pp[(size_t)row * D + nt * 32 + l32] = accQ[i][r];
          }
        }
      }
      if constexpr (ORDERED) {
        fence_release_agent();
        __syncthreads();
        if (tid == 0) store_release_agent(cnt, (uint32_t)rank + 1u);
      } else {
        __syncthreads();
      }
    }
    if (cur_kv >= 0) flush_dkdv();

    // next unit
    if (a.dynamic) {
      if (tid == 0)
        sUnit = (int)__hip_atomic_fetch_add(&a.header[1], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + (int)gridDim.x;
      __syncthreads();
      unit = sUnit;
      __syncthreads();
    } else {
      unit += a.p_eff;
    }
  }
}

// ------------------------------------------------------------ dispatch

template <typename T, int D, int BC, int BR>
static void* pick(bool causal, bool ordered) {
  if (causal)
    return ordered ? (void*)bwd_kernel<T, D, BC, BR, true, true>
                   : (void*)bwd_kernel<T, D, BC, BR, true, false>;
  return ordered ? (void*)bwd_kernel<T, D, BC, BR, false, true>
                 : (void*)bwd_kernel<T, D, BC, BR, false, false>;
}

static void* select_bwd(int dtype, int d, bool causal, bool ordered, int* threads) {
  if (dtype == 1 && d == 128) { *threads = 256; return pick<bf16_t, 128, 128, 64>(causal, ordered); }
  if (dtype == 1 && d == 64) { *threads = 256; return pick<bf16_t, 64, 128, 64>(causal, ordered); }
  if (dtype == 0 && d == 64) { *threads = 128; return pick<float, 64, 64, 64>(causal, ordered); }
  if (dtype == 0 && d == 128) { *threads = 128; return pick<float, 128, 64, 32>(causal, ordered); }
  return nullptr;
}

void bwd_tiles(int dtype, int d, int* bc, int* br) {
  if (dtype == 1) { *bc = 128; *br = 64; }
  else { *bc = 64; *br = (d == 128) ? 32 : 64; }
}

hipError_t bwd_max_coresident(int dtype, int d, bool causal, bool ordered, int* blocks) {
  int threads = 0;
  void* f = select_bwd(dtype, d, causal, ordered, &threads);
  if (!f) return hipErrorInvalidValue;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, threads, 0);
  if (e != hipSuccess) return e;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_bwd(int dtype, int d, bool causal, bool ordered, const BwdArgs& a, int grid,
                      hipStream_t stream) {
  int threads = 0;
  void* f = select_bwd(dtype, d, causal, ordered, &threads);
  if (!f) return hipErrorInvalidValue;
  BwdArgs copy = a;
  void* args[] = {&copy};
  // Cooperative launch: the runtime refuses a grid whose workgroups cannot
  // all be resident, which the ordered waits rely on.
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(threads), args, 0, stream);
}

}  // namespace dash
