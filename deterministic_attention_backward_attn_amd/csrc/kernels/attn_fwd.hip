// Attention forward for gfx950: O = softmax(s Q K^T) V and LSE.
//
// It produces the O and LSE that the backward consumes.  One workgroup per
// (head, 32*NW query rows); wave w owns 32 query rows and keeps them in
// registers as the B operand of S^T = K Q^T, so each lane holds one query
// column and the row statistics (max, sum) need one exchange between the
// two lane halves.  Keys/values stream through LDS in tiles of BN rows with
// an online softmax; O^T = V^T P^T accumulates with the query on lanes, so
// the per-row rescale is a per-lane scalar.  LSE is the natural log of the
// row's sum of exp(s * score).  Masked kernels visit only key tiles that
// can hold a visible key (element bounds lo <= i - j <= hi, and the tile
// liveness of a block mask) and hide the rest per element; a row that sees
// no key gets O = 0 and LSE = -inf.
#include "common.hpp"
#include "launch.hpp"

namespace dash {

template <typename T, int D, int NW, int BN, bool MASKED>
__global__ void __launch_bounds__(NW * 64, 1) fwd_kernel(FwdArgs a) {
  using E = Elt<T>;
  using frag = typename E::frag;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KPL = E::KPL;
  constexpr int KSTEP = E::KSTEP;
  constexpr int VEC = E::VEC;
  constexpr int DK = D / KSTEP;
  constexpr int MT = BN / 32;   // 32-row tiles of a key tile
  constexpr int MD = D / 32;    // 32-row tiles of O^T
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LK = D + PAD;   // sK row stride ([kv][d])
  constexpr int LV = BN + PAD;  // sVt row stride ([d][kv])

  __shared__ __align__(16) T sK[BN * LK];
  __shared__ __align__(16) T sVt[D * LV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int N = a.N;
  const int n_qb = N / BM;
  const int head = blockIdx.x / n_qb;
  const int q0 = (blockIdx.x - head * n_qb) * BM;
  const size_t hoff = (size_t)head * N * D;
  const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
  const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
  const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
  const int qi = q0 + 32 * w + l32;  // this lane's query row

  frag Qreg[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) Qreg[ks] = load_frag(Qg + (size_t)qi * D + ks * KSTEP + hh * KPL);

  f32x16 accO[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) accO[md] = zero16();
  float m = -INFINITY;  // running max of s*score*log2(e)
  float l = 0.f;        // running sum of exp2(. - m)

  // key tiles that can hold a visible key for rows q0 .. q0 + BM - 1
  int j_lo = 0, j_hi = N / BN;
  if (MASKED) {
    const int k_min = q0 - a.mask_hi;             // i - j <= hi
    const int k_max = q0 + BM - 1 - a.mask_lo;    // i - j >= lo
    j_lo = k_min > 0 ? k_min / BN : 0;
    j_hi = k_max < N - 1 ? k_max / BN + 1 : N / BN;
  }
  for (int j = j_lo; j < j_hi; ++j) {
    const int k0 = j * BN;
    // block mask: skip tiles of dead pairs (uniform: BM rows are one tile)
    if (MASKED && a.live && !a.live[(size_t)(q0 / a.tile) * a.n_tiles + k0 / a.tile]) continue;
    __syncthreads();
    for (int c = tid; c < BN * D / VEC; c += NT) {
      const int row = c / (D / VEC);
      const int col = (c % (D / VEC)) * VEC;
      *reinterpret_cast<uint4*>(&sK[row * LK + col]) =
          *reinterpret_cast<const uint4*>(Kg + (size_t)(k0 + row) * D + col);
      const uint4 rv = *reinterpret_cast<const uint4*>(Vg + (size_t)(k0 + row) * D + col);
      const T* e = reinterpret_cast<const T*>(&rv);
#pragma unroll
      for (int t = 0; t < VEC; ++t) sVt[(col + t) * LV + row] = e[t];
    }
    __syncthreads();

    f32x16 accS[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) accS[mt] = zero16();
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        accS[mt] = E::mma(load_frag(&sK[(mt * 32 + l32) * LK + ks * KSTEP + hh * KPL]), Qreg[ks],
                          accS[mt]);
    }
    // accS[mt][r]: key k0 + mt*32 + crow(r, hh), query qi
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s2 = accS[mt][r] * a.scale_log2;
        if (MASKED) {
          const int dd = qi - (k0 + mt * 32 + crow(r, hh));
          if (dd < a.mask_lo || dd > a.mask_hi) s2 = -INFINITY;
        }
        accS[mt][r] = s2;
        mx = fmaxf(mx, s2);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    // while a row has seen no key its max stays -inf: subtract 0 instead
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(accS[mt][r] - m_use);
        accS[mt][r] = p;
        ps += p;
      }
    }
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int md = 0; md < MD; ++md) accO[md] *= alpha;

    // O^T += V^T P^T, contraction over this key tile
#pragma unroll
    for (int c = 0; c < BN / KSTEP; ++c) {
      constexpr int CPM = 32 / KSTEP;
      const int mt = c / CPM;
      const int cc = c % CPM;
      frag pb;
      if constexpr (KPL == 8) {
        float tp[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) tp[s] = accS[mt][8 * cc + s];
        pb = pack_bf16x8(tp);
      } else {
        pb = accS[mt][cc];
      }
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int drow = md * 32 + l32;
        frag va;
        if constexpr (KPL == 8) {
          const int base = drow * LV + mt * 32 + 16 * cc + 4 * hh;
          const u16x4 v0 = *reinterpret_cast<const u16x4*>(&sVt[base]);
          const u16x4 v1 = *reinterpret_cast<const u16x4*>(&sVt[base + 8]);
          u16x8 u;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            u[s] = v0[s];
            u[s + 4] = v1[s];
          }
          va = __builtin_bit_cast(bf16x8, u);
        } else {
          va = load_frag(&sVt[drow * LV + mt * 32 + crow(cc, hh)]);
        }
        accO[md] = E::mma(va, pb, accO[md]);
      }
    }
  }

  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  T* Og = reinterpret_cast<T*>(a.o) + hoff;
#pragma unroll
  for (int md = 0; md < MD; ++md) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dcol = md * 32 + crow(r, hh);
      Og[(size_t)qi * D + dcol] = E::from_f32(accO[md][r] * inv_l);
    }
  }
  if (hh == 0)
    a.lse[(size_t)head * N + qi] = l > 0.f ? (m + log2f(l)) * (1.0f / kLog2e) : -INFINITY;
}

// max(x of this lane, x of lane l ^ 32): v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second, so
// with x in both the two results hold, per lane, x and the other half's x.
// A VALU operation (no LDS traffic, unlike a shuffle).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// bf16 forward.  A workgroup owns NW x 32QN query rows: NW waves x QN
// 32-query column tiles.  With QN = 2 every K / V fragment read from LDS
// feeds two MFMAs and a wave needs more than half a SIMD's registers (one
// wave per SIMD: its softmax leaves the matrix core idle); with QN = 1 and
// 8 waves two waves share each SIMD at 256 registers, and one wave's
// softmax runs beside the other's MFMAs, for twice the LDS reads per MFMA
// (16K causal d = 128: 2.80 -> 2.46 ms; d = 64 and the block-mask kernel
// lose, 6.0 -> 7.1 and 0.85 -> 0.94 ms, and keep QN = 2).  Key and value
// tiles of 64 rows stay row-major in LDS (XOR
// swizzled, double buffered) and are prefetched into registers one tile
// ahead, so a tile costs one workgroup barrier.  S^T = K Q^T with K from LDS
// (A operand) and Q^T in registers (B); O^T = V^T P^T with V^T from the
// transposing LDS read (A) and P^T taken straight from the S^T accumulators
// (B), their key order matching the accumulator's row order.  The query is
// on lanes: row statistics need one exchange between the lane halves and
// the rescale of O^T is a per-lane scalar.  Waves skip key tiles their rows
// cannot see and mask elements only on tiles that cross a mask bound.
template <int D, bool MASKED, int NW, int QN>
__global__ void __launch_bounds__(NW * 64, QN == 1 ? 8 / NW : 1) fwd_bf16_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int WR = 32 * QN;              // query rows per wave
  constexpr int BM = NW * WR;              // query rows per workgroup
  constexpr int BN = 64;                   // keys per tile
  constexpr int DK = D / 16;               // MFMA steps over d
  constexpr int MT = BN / 32;              // 32-key tiles
  constexpr int MD = D / 32;               // 32-row tiles of O^T
  constexpr int CPT = BN * D / 8 / NT;     // 16-byte chunks per thread per tensor
  static_assert(CPT >= 1 && CPT * 8 * NT == BN * D, "tile staging");
  __shared__ __align__(16) bf16_t sK[2][BN * D];
  __shared__ __align__(16) bf16_t sV[2][BN * D];
  // block-mask liveness of the (at most 2) query tiles this workgroup covers
  constexpr int kMaxLive = 2048;
  __shared__ uint8_t sLive[MASKED ? 2 * kMaxLive : 1];
  const auto kix = [](int r, int c) { return r * D + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // a scalar
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int j16 = lane & 15;
  const int gcol = 16 * ((lane >> 4) & 1);
  const int N = a.N;
  const int n_qb = (N + BM - 1) / BM;
  // the heaviest query blocks first (under a causal mask work grows with
  // the block index); heads vary fastest
  const int qb = n_qb - 1 - (int)(blockIdx.x / (unsigned)a.BH);
  const int head = (int)(blockIdx.x % (unsigned)a.BH);
  const int q0 = qb * BM;
  const int q_end = q0 + BM < N ? q0 + BM : N;
  const size_t hoff = (size_t)head * N * D;
  const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + hoff;
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + hoff;
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + hoff;
  // the tile liveness rows of this workgroup's query tiles (tile = 128 rows)
  const int qt0 = q0 / (MASKED ? a.tile : 1);
  if (MASKED && a.live) {
    for (int i = tid; i < 2 * a.n_tiles; i += NT) {
      const int r = qt0 + i / a.n_tiles;
      sLive[i] = r < a.n_tiles ? a.live[(size_t)r * a.n_tiles + i % a.n_tiles] : 0;
    }
    __syncthreads();
  }

  // Does wave v (rows q0 + v*WR ...) need key tile j, and must it mask
  // elements there?  i - j over the pair spans [qv - k0 - 63, qv + WR-1 - k0].
  const auto need = [&](int v, int j, bool* emask) {
    const int qv = q0 + v * WR;
    if (qv >= N) return false;
    const int k0 = j * BN;
    if (!MASKED) {
      *emask = false;
      return true;
    }
    const int dmin = qv - (k0 + BN - 1), dmax = qv + WR - 1 - k0;
    if (dmax < a.mask_lo || dmin > a.mask_hi) return false;
    if (a.live && !sLive[(qv / a.tile - qt0) * a.n_tiles + k0 / a.tile]) return false;
    *emask = dmin < a.mask_lo || dmax > a.mask_hi;
    return true;
  };
  const auto need_any = [&](int j) {
    bool e, any = false;
#pragma unroll
    for (int v = 0; v < NW; ++v) any = any || need(v, j, &e);
    return any;
  };
  int j_lo = 0, j_hi = N / BN;
  if (MASKED) {
    const int k_min = q0 - a.mask_hi;
    const int k_max = q_end - 1 - a.mask_lo;
    j_lo = k_min > 0 ? k_min / BN : 0;
    j_hi = k_max < N - 1 ? k_max / BN + 1 : N / BN;
  }
  // Without a block mask every key tile in [j_lo, j_hi) is needed by some
  // row of the workgroup (each row sees one contiguous key range, and the
  // ranges of consecutive rows overlap or adjoin), so the next tile is the
  // following one; a block mask needs the search.
  const auto next_tile = [&](int j) {
    if (!(MASKED && a.live)) return j + 1 < j_hi ? j + 1 : j_hi;
    for (++j; j < j_hi; ++j)
      if (need_any(j)) return j;
    return j_hi;
  };

  const int qw = q0 + w * WR;
  bf16x8 Qreg[QN][DK];
#pragma unroll
  for (int nt = 0; nt < QN; ++nt) {
    const int row = qw + nt * 32 + l32 < N ? qw + nt * 32 + l32 : N - 1;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) Qreg[nt][ks] = load_frag(Qg + (size_t)row * D + ks * 16 + hh * 8);
  }
  // Settle the query loads here: the fragments pass through an empty asm,
  // so inside the loop they no longer count as outstanding loads (vector
  // memory completions are counted in order, and a wait for them there
  // would also wait for the key/value prefetch issued after them).
#pragma unroll
  for (int nt = 0; nt < QN; ++nt)
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) asm volatile("" : "+v"(Qreg[nt][ks]));
  f32x16 accO[MD][QN];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nt = 0; nt < QN; ++nt) accO[md][nt] = zero16();
  float m_run[QN], l_run[QN];
#pragma unroll
  for (int nt = 0; nt < QN; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  u32x4 pk[CPT], pv[CPT];
  const auto fetch = [&](int j) {
    const int k0 = j * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const size_t off = (size_t)(k0 + c / (D / 8)) * D + (c % (D / 8)) * 8;
      pk[i] = *reinterpret_cast<const u32x4*>(Kg + off);
      pv[i] = *reinterpret_cast<const u32x4*>(Vg + off);
    }
  };
  const auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int o = kix(c / (D / 8), (c % (D / 8)) * 8);
      *reinterpret_cast<u32x4*>(&sK[buf][o]) = pk[i];
      *reinterpret_cast<u32x4*>(&sV[buf][o]) = pv[i];
    }
  };

  int j = next_tile(j_lo - 1);
  int jn = j_hi;
  if (j < j_hi) {
    fetch(j);
    stage(0);
    jn = next_tile(j);
    if (jn < j_hi) fetch(jn);
  }
  __syncthreads();
  // One key tile; the loop below alternates the two buffers with the
  // buffer index a constant in each copy, so that every LDS address is a
  // per-lane offset plus an immediate.
  const auto tile = [&](auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    bool emask = false;
    if (need(w, j, &emask)) {
      const bf16_t* cK = sK[buf];
      const bf16_t* cV = sV[buf];
      const int k0 = j * BN;
      f32x16 accS[MT][QN];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < QN; ++nt) accS[mt][nt] = zero16();
      // K fragments in groups of KG steps: a group's LDS reads are issued
      // together, then its MFMAs (the barriers keep the compiler from
      // placing each read right before its consumer)
      constexpr int KG = DK / 2;
#pragma unroll
      for (int g = 0; g < DK / KG; ++g) {
        bf16x8 kf[KG][MT];
#pragma unroll
        for (int k2 = 0; k2 < KG; ++k2)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            kf[k2][mt] = load_frag(&cK[kix(mt * 32 + l32, (g * KG + k2) * 16 + hh * 8)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k2 = 0; k2 < KG; ++k2)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < QN; ++nt)
              accS[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  kf[k2][mt], Qreg[nt][g * KG + k2], accS[mt][nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // online softmax per query (lane) column; P packed to bf16 pairs
      uint32_t pP[MT][QN][8];
#pragma unroll
      for (int nt = 0; nt < QN; ++nt) {
        if (MASKED && emask) {
          // i - j of register r: qi - k0 - mt*32 - crow(r, h)
          const int base = qw + nt * 32 + l32 - k0 - 4 * hh;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int dd = base - mt * 32 - ((r >> 2) << 3) - (r & 3);
              accS[mt][nt][r] = (dd < a.mask_lo || dd > a.mask_hi) ? -INFINITY : accS[mt][nt][r];
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, accS[mt][nt][r]);
        mx = max_halves(mx);
        // Lazy rescaling: the running max (exp2 domain; scale > 0 keeps the
        // order) moves, and O^T and the sum are rescaled, only when some
        // query of the wave gained more than 2^8 over it; otherwise P is
        // taken against the stale max (at most 2^8, exact in the final
        // normalisation by the sum).
        const float cand = fmaxf(m_run[nt], mx * a.scale_log2);
        if (__builtin_amdgcn_ballot_w64(cand > m_run[nt] + 8.0f) != 0) {
          const float c_use = cand == -INFINITY ? 0.f : cand;
          const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - c_use);
          m_run[nt] = cand;
          l_run[nt] *= alpha;
#pragma unroll
          for (int md = 0; md < MD; ++md) accO[md][nt] *= alpha;
        }
        // a row that has seen no key yet keeps max -inf: subtract 0 instead
        const float m_use = m_run[nt] == -INFINITY ? 0.f : m_run[nt];
        float ps = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(accS[mt][nt][r], a.scale_log2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(accS[mt][nt][r + 1], a.scale_log2, -m_use));
            pP[mt][nt][r / 2] = pack2_bf16(p0, p1);
            ps += p0 + p1;
          }
        // each lane half keeps the sum over its own keys (the halves share
        // the running max); they are added once at the end
        l_run[nt] += ps;
      }
      // O^T += V^T P^T over this tile's keys, 16 keys per step: keys
      // mt*32 + 16cc + 4h + {0..3} and + 8 + {0..3} (the accumulator's rows)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x8 pb[QN];
#pragma unroll
          for (int nt = 0; nt < QN; ++nt)
            pb[nt] = __builtin_bit_cast(bf16x8, make_uint4(pP[mt][nt][4 * cc], pP[mt][nt][4 * cc + 1],
                                                           pP[mt][nt][4 * cc + 2],
                                                           pP[mt][nt][4 * cc + 3]));
          const int r0 = mt * 32 + 16 * cc + 4 * hh;
          bf16x8 va[MD];
#pragma unroll
          for (int md = 0; md < MD; ++md) va[md] = tr_frag(cV, kix, r0, r0 + 8, md * 32 + gcol, j16);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int nt = 0; nt < QN; ++nt)
              accO[md][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[md], pb[nt], accO[md][nt],
                                                                     0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the prefetched tile into the other buffer (last read before the
    // previous barrier), then the next prefetch
    int jnn = j_hi;
    if (jn < j_hi) {
      stage(buf ^ 1);
      jnn = next_tile(jn);
      if (jnn < j_hi) fetch(jnn);
    }
    __syncthreads();
    j = jn;
    jn = jnn;
  };
  while (j < j_hi) {
    tile(std::integral_constant<int, 0>{});
    if (j >= j_hi) break;
    tile(std::integral_constant<int, 1>{});
  }

  if (qw >= N) return;
  bf16_t* Og = reinterpret_cast<bf16_t*>(a.o) + hoff;
#pragma unroll
  for (int nt = 0; nt < QN; ++nt) l_run[nt] += __shfl_xor(l_run[nt], 32);
#pragma unroll
  for (int nt = 0; nt < QN; ++nt) {
    const int qi = qw + nt * 32 + l32;
    const float inv_l = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack2_bf16(accO[md][nt][4 * g] * inv_l, accO[md][nt][4 * g + 1] * inv_l);
        u.y = pack2_bf16(accO[md][nt][4 * g + 2] * inv_l, accO[md][nt][4 * g + 3] * inv_l);
        *reinterpret_cast<uint2*>(Og + (size_t)qi * D + md * 32 + 8 * g + 4 * hh) = u;
      }
    if (hh == 0)
      a.lse[(size_t)head * N + qi] =
          l_run[nt] > 0.f ? (m_run[nt] + log2f(l_run[nt])) * (1.0f / kLog2e) : -INFINITY;
  }
}

// Block masks: workgroups of one query tile (2 waves, 128 rows), so the
// waves of a workgroup see the same live key tiles; two such workgroups
// share a compute unit.  Otherwise 256 rows: d = 128 in 8 waves of 32 rows
// (two per SIMD), d = 64 in 4 waves of 64.
template <int D>
static hipError_t go_fwd_bf16(bool masked, const FwdArgs& a, hipStream_t s) {
  const int nw = a.live ? 2 : 4;
  if (a.live && 64 * nw != a.tile) return hipErrorInvalidValue;
  const long blocks = (long)((a.N + 64 * nw - 1) / (64 * nw)) * a.BH;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  constexpr int NW = D == 128 ? 8 : 4, QN = D == 128 ? 1 : 2;
  if (a.live) hipLaunchKernelGGL((fwd_bf16_kernel<D, true, 2, 2>), grid, dim3(128), 0, s, a);
  else if (masked) hipLaunchKernelGGL((fwd_bf16_kernel<D, true, NW, QN>), grid, dim3(NW * 64), 0, s, a);
  else hipLaunchKernelGGL((fwd_bf16_kernel<D, false, NW, QN>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BN>
static hipError_t go_fwd(bool masked, const FwdArgs& a, hipStream_t s) {
  // one workgroup per (head, query block); the block is one tile
  if (32 * NW != a.tile) return hipErrorInvalidValue;
  const long blocks = (long)(a.N / (32 * NW)) * a.BH;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  if (masked) hipLaunchKernelGGL((fwd_kernel<T, D, NW, BN, true>), grid, dim3(NW * 64), 0, s, a);
  else hipLaunchKernelGGL((fwd_kernel<T, D, NW, BN, false>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int d, bool masked, const FwdArgs& a, hipStream_t stream) {
  if (dtype == 1 && d == 128) return go_fwd_bf16<128>(masked, a, stream);
  if (dtype == 1 && d == 64) return go_fwd_bf16<64>(masked, a, stream);
  if (dtype == 0 && d == 64) return go_fwd<float, 64, 2, 64>(masked, a, stream);
  if (dtype == 0 && d == 128) return go_fwd<float, 128, 2, 64>(masked, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dash
