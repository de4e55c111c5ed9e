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
  if (dtype == 1 && d == 128) return go_fwd<bf16_t, 128, 4, 64>(masked, a, stream);
  if (dtype == 1 && d == 64) return go_fwd<bf16_t, 64, 4, 64>(masked, a, stream);
  if (dtype == 0 && d == 64) return go_fwd<float, 64, 2, 64>(masked, a, stream);
  if (dtype == 0 && d == 128) return go_fwd<float, 128, 2, 64>(masked, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dash
