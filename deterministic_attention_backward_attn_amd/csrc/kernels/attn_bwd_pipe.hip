// Deterministic attention backward, two-stage pipeline (bf16, d = 128 with
// Q sub-tiles of 32 rows, d = 64 with Q sub-tiles of 64 rows).
//
// The same method, schedules, tables and ordered dQ hand-off as the
// one-wave-per-slice kernel (attn_bwd.hip), with the work of each 32-row KV
// slice split into two stages that run one Q sub-tile apart on the two
// waves sharing a SIMD (8 waves per workgroup, at most 256 registers each):
//
//   stage A (waves 0..3: K and V fragments and the dV accumulator in
//     registers), sub-tile t: S = Q K^T, dP = dO V^T, P = exp(s S - LSE)
//     (masked), dS = P (dP - delta), dV += P^T dO; dS^T to LDS; loads the
//     next Q/dO sub-tile straight into LDS;
//   stage B (waves 4..7: the dK accumulator and K^T fragments), sub-tile
//     t - 1: dK += dS^T Q, dQ_part^T = K^T dS^T, and the ordered add of
//     dQ_part into the fp32 accumulator.
//
// Every input of stage B was written by stage A one period earlier, so one
// workgroup barrier per period is the only synchronisation: within a period
// the two waves of a SIMD never wait for each other, and the matrix core
// runs B's products while A computes its exponentials.  The ordered add's
// memory round trips (counter read, accumulator read, store, hand-off) are
// issued only by the B waves, whose vector-memory queue holds nothing else,
// so a wait for one of them never waits for a prefetch (vector-memory
// operations of a wave complete in issue order).  Results are
// bit-identical to the other layouts: every product, exponential and add is
// computed with the same operands in the same order.
//
// The ordered add (explainer section 1, a fixed accumulation order for dQ)
// keeps the other kernel's protocol: wave B of slice s owns one 32 x 32
// block of the sub-tile's dQ (d = 128: columns [32s, 32s+32); d = 64: Q
// rows [32 (s / 2), +32), columns [32 (s % 2), +32)) in every workgroup and
// hands off to slice s of the next contributor through the sub-tile's
// counter for s.  Its timing per period
// (B processing sub-tile g):
//   1. the counter value read one period earlier shows whether this
//      contributor's turn has come; if it has not, the previous add is
//      released first (a wave never waits while holding an unreleased add)
//      and the counter is polled;
//   2. the accumulator reads for sub-tile g are issued (out of range, reading
//      nothing, for the first contributor), then the counter read for g + 1;
//   3. after the dK product the previous add is released: a wait until its
//      stores completed (exactly the five operations issued after them may
//      still be outstanding), then the counter store;
//   4. after the dQ product the partial is transposed through this wave's LDS
//      area, added to the accumulator values and stored (the last contributor
//      writes the scaled dQ instead).
#include "common.hpp"
#include "launch.hpp"
#include "placement.hpp"

namespace dash {

// Direct global -> LDS loads (lane i of a 16-byte load writes LDS bytes
// [16 i, 16 i + 16) above the LDS address in M0, of a 4-byte load [4 i,
// 4 i + 4)), written as assembly so that the compiler neither counts them in
// its own waits nor makes later reads of other LDS buffers wait for them:
// the caller waits for them (vmcnt) before the barrier after which they are
// read.  No register receives data; the leading no-ops cover a scalar
// operand written by a vector instruction just before.  M0 is written here
// and used by no other instruction of this kernel.
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma_b128(const void* gbase, uint32_t voff, const void* lds) {
  // the base address and the LDS address are the same in every lane
  // (readfirstlane returns a signed int: widen through uint32_t, never
  // sign-extend the low half)
  const uint64_t b = (uint64_t)(uintptr_t)gbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lds));
  asm volatile(
      "s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
      :: "v"(voff), "s"(bs), "s"(ls) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* gaddr, const void* lds) {
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lds));
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\tglobal_load_lds_dword %0, off"
               :: "v"(gaddr), "s"(ls) : "memory", "m0");
}

// `p` advanced by `bytes`
template <typename P>
__device__ __forceinline__ P* at(P* p, uint32_t bytes) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(const_cast<void*>(static_cast<const void*>(p))) + bytes);
}
// Transposing fragment read (as tr_frag) from two given addresses: K slots
// 0..3 from `pa`, 4..7 from `pb`.
__device__ __forceinline__ bf16x8 tr_frag_at(const bf16_t* pa, const bf16_t* pb) {
  const u16x4 x = lds_tr16(pa);
  const u16x4 y = lds_tr16(pb);
  u16x8 u;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u[s] = x[s];
    u[s + 4] = y[s];
  }
  return __builtin_bit_cast(bf16x8, u);
}

template <int D, bool MASKED, bool ORDERED, bool DEBUG>
__global__ void __launch_bounds__(512, 1) bwd_pipe_kernel(BwdArgs a) {
  using T = bf16_t;
  using E = Elt<T>;
  using frag = typename E::frag;
  static_assert(D == 128 || D == 64, "head dim");
  // Q sub-tiles of 32 rows at d = 128, 64 at d = 64: the same MFMA work per
  // period (A 24, B 16 products) and the same 8 KB per staged sub-tile
  constexpr int BC = 128, BR = D == 128 ? 32 : 64;
  constexpr int QT = BR / 32;           // 32-row Q tiles per sub-tile
  constexpr int CS = BR / 16;           // MFMA steps over a sub-tile's Q rows
  constexpr int NW = 4;                 // KV slices (counter layout: one per slice)
  constexpr int NT = 512;
  constexpr int NA = 256;               // threads of stage A
  constexpr int RHO = BC / BR;          // Q sub-tiles per Q block
  constexpr int KPL = 8, KSTEP = 16, VEC = 8;
  constexpr int DK = D / KSTEP;         // 8 MFMA steps over d
  constexpr int KK = BC / KSTEP;        // 8 MFMA steps over the KV tile
  constexpr int NTD = D / 32;           // column tiles over d
  constexpr int LQ = D;
  constexpr int LS = BR;                // row stride of sdSt ([kv][q], swizzled)
  constexpr int CPT = BR * D / VEC / NA;  // 16-byte chunks per A thread per tensor (2)
  static_assert(CPT == 2, "sub-tile load: two 1 KB loads per A wave and tensor");
  static_assert(CS * NTD == KK, "dK steps pair with the dQ operand reads");
  // B wave w: dQ columns [32 DT, 32 DT + 32) of the sub-tile's Q rows
  // [32 QW, 32 QW + 32) (d = 128: DT = w; d = 64: DT = w % 2, QW = w / 2)

  // Q / dO / LSE / delta sub-tiles: sub-tile g in buffer g % 4 (A reads t,
  // B reads t - 1, the loads of t + 1 and t + 2 in flight).  dS^T of
  // sub-tile g in buffer g % 2 (A writes t, B reads t - 1).
  constexpr int NQB = 4;
  constexpr int LR = 32;
  // One LDS block, so that the layout is fixed: a dO buffer lies 32 KB
  // after the Q buffer of the same index, a distance the LDS instructions
  // take as an immediate offset (one address register per Q/dO pair of
  // operand reads).
  struct __align__(16) Lds {
    T q[NQB][BR * LQ];
    T dO[NQB][BR * LQ];
    T dSt[2][BC * LS];
    T k[BC * LQ];
    // LSE * log2(e) in [0, BR), delta in [BR, 2 BR) of each buffer
    float stat[NQB][2 * BR];
    float row[ORDERED ? NW : 1][ORDERED ? 32 * LR : 4];
    int2 items[kMaxUnitItems];
    int unit;
    int place[5];
  };
  __shared__ Lds L;
  auto& sQ = L.q;
  auto& sdO = L.dO;
  auto& sdSt = L.dSt;
  auto& sK = L.k;
  auto& sStat = L.stat;
  auto& sItems = L.items;
  auto& sRow = L.row;
  auto& sUnit = L.unit;
  auto& sPlace = L.place;
  // a dO buffer lies this many bytes after the Q buffer of the same index
  constexpr uint32_t kQtoDO = (uint32_t)(offsetof(Lds, dO) - offsetof(Lds, q));
  const auto qix = [](int r, int c) { return r * LQ + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7); };
  // dS^T rows: 8-byte unit u (4 elements) of row r at unit u ^ dsw(r), so
  // that the 16 lanes of a write step (16 consecutive rows, one unit), the
  // 32 lanes of a row read (32 consecutive rows) and the transposing reads
  // (4 rows, 64 bytes of each) each touch distinct banks
  const auto dsw = [](int r) {
    if constexpr (BR == 32) return ((r >> 1) & 7) ^ ((r >> 4) & 1);
    else return ((r & 1) ^ ((r >> 4) & 1)) | (((r >> 2) & 1) << 1) | (((r >> 3) & 1) << 2) | (((r >> 1) & 1) << 3);
  };
  const auto six = [=](int r, int c) { return r * LS + ((((c >> 2) ^ dsw(r)) << 2) | (c & 3)); };
  // partial rows, 16-byte chunk c of row r at chunk c ^ (r % 8) (measured
  // 2 % faster for descending than c ^ (r / 2 % 8))
  const auto rix = [](int r, int c) { return r * LR + (((c >> 2) ^ (r & 7)) << 2) + (c & 3); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, a scalar
  const bool isA = wv < NW;
  const int w = wv & 3;                 // KV slice
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int j16 = lane & 15;
  const int gcol = 16 * ((lane >> 4) & 1);
  const int N = a.N;
  const int n_sub = N / BR;
  uint32_t* status = a.header;
  const uint32_t spin_limit = a.spin_limit;
  const int kvl = 32 * w + l32;         // this lane's KV row within the tile
  const int DT = w % NTD, QW = w / NTD;

  uint64_t st_wait = 0, st_waits = 0, st_spun = 0;
  const uint64_t st_t0 = (DEBUG && a.wait_stats) ? (uint64_t)clock64() : 0;
  // phase timer (test hook, debug instantiation only): lane 0 of each wave
  // adds the shader-clock cycles since the previous mark to the phase that
  // just ended.  Stage A: 0 item decode, KV tile changes and the next
  // sub-tile's loads, 1 S and dP products, 2 softmax and dS, 3 dV product,
  // 4 barrier.  Stage B: 0 item decode and KV tile changes, 1 turn check and
  // accumulator reads, 2 dK product, 3 hand-off, 4 dQ product, 5 ordered
  // add, 6 barrier.
  uint64_t ph[8] = {};
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
  // (read from LDS, the same in every lane: scalar registers)
  const int grp = __builtin_amdgcn_readfirstlane(pl.grp);
  const int n_grp = __builtin_amdgcn_readfirstlane(pl.n_grp);
  const int li = __builtin_amdgcn_readfirstlane(pl.li);
  const int W = __builtin_amdgcn_readfirstlane(pl.W);
  const bool grouped = pl.grouped;
  const int BH = a.total_units / U;
  const int hg = (BH - grp + n_grp - 1) / n_grp;
  const int n_units = hg * U;
  const int stride_static = grouped ? (W / U) * U : a.p_eff;
  uint32_t* work_counter = grouped ? &a.header[20 + grp] : &a.header[1];
  const int unit0 = (a.dynamic == 0 && li >= stride_static) ? n_units : li;

  // Per-lane byte offsets of the transposing reads of a Q or dO sub-tile
  // (rows 4 hh + 8 h + j16 / 4, columns 32 nt + gcol + 4 (j16 % 4)); rows
  // 16 further lie 16 LQ elements further (the swizzle repeats every 16
  // rows), a constant offset.
  uint32_t oT[2][NTD];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt)
      oT[h][nt] = (uint32_t)(2 * qix(4 * hh + 8 * h + (j16 >> 2), nt * 32 + gcol + 4 * (j16 & 3)));
  const auto tr_sub = [&](const T* base, int cc, int nt) {
    return tr_frag_at(at(base, oT[0][nt] + 2 * 16 * cc * LQ), at(base, oT[1][nt] + 2 * 16 * cc * LQ));
  };
  // ... and of dS^T (rows 8 hh + j16 / 4, columns gcol + 4 (j16 % 4)), the
  // rows of KV step i and the second half's 4 rows a constant further
  // (the swizzle of rows 16 i + r' depends on i only through i % 2, and
  // rows 4 further need their own offsets)
  uint32_t oF[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      oF[p][e] = (uint32_t)(2 * six(16 * p + 8 * hh + 4 * e + (j16 >> 2), 32 * QW + gcol + 4 * (j16 & 3)) -
                            2 * 16 * p * LS);
  // dS^T writes (Q tile m: unit 8 m + 2 gq + hh of row kvl) and row reads
  // (units 4 cc + hh and 4 cc + hh + 2), byte offsets within a buffer
  uint32_t oDw[QT][4], oDr[CS][2];
#pragma unroll
  for (int m = 0; m < QT; ++m)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) oDw[m][gq] = (uint32_t)(2 * six(kvl, 32 * m + 8 * gq + 4 * hh));
#pragma unroll
  for (int cc = 0; cc < CS; ++cc)
#pragma unroll
    for (int e = 0; e < 2; ++e) oDr[cc][e] = (uint32_t)(2 * six(kvl, 16 * cc + 4 * hh + 8 * e));

  // One copy of the unit loop per stage, so that each stage's registers are
  // allocated for its own values only; both copies pass the same barriers
  // in the same order.  Stage B has one copy per accumulator cache policy
  // (XL: the head's contributors share one XCD's L2), so that its memory
  // operations are not split over branches.
  auto run = [&](auto stage_tag, auto xl_tag) {
    constexpr bool IS_A = decltype(stage_tag)::value;
    constexpr bool XL = decltype(xl_tag)::value;
    constexpr int POL = XL ? kXcdCoherent : kCoherent;
    int unit = unit0;
    while (unit < n_units) {
      const int hq = a.unit_major ? unit % hg : unit / U;
      const int lu = a.unit_major ? unit / hg : unit - hq * U;
      const int head = grp + n_grp * hq;
      const size_t hoff = (size_t)head * N * D;
      const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
      const T* dOg = reinterpret_cast<const T*>(a.dout) + hoff;
      const int it0 = a.unit_off[lu];
      const int n_items = a.unit_off[lu + 1] - it0;  // <= kMaxUnitItems (checked by the host)
      const int n_steps = n_items * RHO;

      // every wave has finished the previous unit (its last reads of the
      // work list included) before the list is overwritten
      __syncthreads();
      for (int i = tid; i < n_items; i += NT) sItems[i] = a.items[it0 + i];
      __syncthreads();

      // work-list entry i, the same in every lane: moved to scalar registers,
      // so that what is derived from it (tile indices, addresses, flags) is
      // computed by scalar instructions
      const auto uniform = [](int2 v) {
        return make_int2(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y));
      };
      // Stage A reads its entries one period before it uses them (into
      // vector registers, made scalar at the start of the period that uses
      // them), so that its periods do not start by waiting for an LDS round
      // trip (stage B doing the same measured slower for naive).  Entry i
      // clamped to the list (the read past its end, at the last period, is
      // never used).
      const auto raw_item = [&](int i) { return sItems[i < n_items ? i : (n_items > 0 ? n_items - 1 : 0)]; };

      if constexpr (IS_A) {
        // ---------------------------------------------------------- stage A
        const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
        const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
        const float* lse_g = a.lse2 + (size_t)head * N;  // LSE * log2(e)
        const float* del_g = a.delta + (size_t)head * N;
        // Sub-tile g into buffer `buf` by direct loads to LDS (no registers:
        // lane i of a 16-byte load writes LDS bytes [16 i, 16 i + 16) of the
        // instruction's 1 KB).  Wave w loads LDS bytes [2048 w, 2048 w + 2048)
        // of sQ and of sdO, i.e. rows RW w .. RW w + RW - 1: lane i of
        // instruction m fills row RW w + RI m + i / (D / 8), 16-byte slot
        // i % (D / 8), which holds the row's global chunk (slot ^ swz(row)).
        // Waves 0 (and 1 at d = 64) also load LSE and delta (one dword per
        // lane).  The loads complete before the barrier that ends the period
        // (the compiler waits for them there).
        constexpr int RW = BR / 4, RI = 512 / D, CPR = D / 8;
        const int wu = __builtin_amdgcn_readfirstlane(w);
        // per-lane element offsets within a sub-tile of the two 16-byte loads
        uint32_t doff[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int row = RW * w + RI * m + lane / CPR;
          doff[m] = (uint32_t)(row * D + ((lane % CPR) ^ swz<D>(row)) * VEC);
        }
        // stat dword 64 wu + lane: LSE of rows < BR, then delta
        const int sidx = 64 * w + lane;
        const bool stat_wave = 64 * wu < 2 * BR;
        const float* stat_src = sidx < BR ? lse_g + sidx : del_g + (sidx < 2 * BR ? sidx - BR : 0);
        auto dma = [&](int qtile, int buf) {
          const int q0 = qtile * BR;
          const T* qs = Qg + (size_t)q0 * D;
          const T* os = dOg + (size_t)q0 * D;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            dma_b128(qs, doff[m] * (uint32_t)sizeof(T), &sQ[buf][(RW * wu + RI * m) * LQ]);
            dma_b128(os, doff[m] * (uint32_t)sizeof(T), &sdO[buf][(RW * wu + RI * m) * LQ]);
          }
          if (stat_wave) dma_b32(stat_src + q0, &sStat[buf][64 * wu]);
        };
        // Wait for this wave's loads of the sub-tile read after the next
        // barrier: only the loads issued after them (4 or 5 when sub-tile
        // t + 2 was staged this period) may stay in flight.
        auto wait_staged = [&](bool newer) {
          if (newer) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
          else __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
        };
        frag Kreg[DK], Vreg[DK];
        f32x16 accdV[NTD];
        int a_kv = -1;
        auto flush_dv = [&]() {
          T* dVg = reinterpret_cast<T*>(a.dv) + hoff;
#pragma unroll
          for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              dVg[(uint32_t)((a_kv * BC + 32 * w + crow(r, hh)) * D + nt * 32 + l32)] =
                  E::from_f32(accdV[nt][r]);
        };
        if (n_steps > 0) dma((uniform(raw_item(0)).x >> 16) * RHO, 0);
        if (n_steps > 1) dma((uniform(raw_item(0)).x >> 16) * RHO + 1, 1);
        // the entry of sub-tile t and that of sub-tile t + 2 (staged at t)
        int2 pf_itm = raw_item(0);
        int2 pf_st = raw_item(2 / RHO);
        wait_staged(n_steps > 1);
        __syncthreads();  // sub-tile 0 in LDS

        for (int t = 0; t <= n_steps; ++t) {
          PHASE(4);
          if (t < n_steps) {
            const int b3 = t % NQB;
            const int b2 = t & 1;
            const int2 itm = uniform(pf_itm);
            const int kv = itm.x & 0xFFFF;
            const int qblk = itm.x >> 16;
            const int rsub = t % RHO;
            if (kv != a_kv) {
              // new KV tile: dV of the previous one is complete; K and V
              // fragments (row 32w + l32, columns 16ks + 8h ..), and K
              // row-major into LDS for stage B's K^T (stage B read the
              // previous tile's K one period after it was written, at least
              // three periods ago)
              if (a_kv >= 0) flush_dv();
              a_kv = kv;
#pragma unroll
              for (int nt = 0; nt < NTD; ++nt) accdV[nt] = zero16();
              const int kv0 = kv * BC;
#pragma unroll
              for (int ks = 0; ks < DK; ++ks) {
                const uint32_t off = (uint32_t)((kv0 + kvl) * D + ks * KSTEP + hh * KPL);
                Kreg[ks] = load_frag(Kg + off);
                Vreg[ks] = load_frag(Vg + off);
              }
#pragma unroll
              for (int ks = 0; ks < DK; ++ks)
                *reinterpret_cast<uint4*>(&sK[qix(kvl, ks * KSTEP + hh * KPL)]) =
                    __builtin_bit_cast(uint4, Kreg[ks]);
              // all of this rare path's loads complete here, so that the
              // products below never wait for the sub-tile loads issued
              // after it
              __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            }
            // sub-tile t + 2 into its buffer (its previous contents, sub-tile
            // t - 2, were last read by stage B in the previous period)
            if (t + 2 < n_steps) dma((uniform(pf_st).x >> 16) * RHO + (t + 2) % RHO, (t + 2) % NQB);
            PHASE(0);
            const T* cQ = sQ[b3];
            const T* cdO = sdO[b3];
            // S and dP of Q tile m (rows 32 m .. 32 m + 31; the swizzle
            // repeats every 16 rows, so tile m lies 32 m LQ elements further)
            f32x16 accS[QT], accP[QT];
#pragma unroll
            for (int m = 0; m < QT; ++m) accS[m] = accP[m] = zero16();
            // in two halves over d: all A fragments of a half are read
            // first, then its MFMAs (the scheduling barriers keep them apart)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              frag qa[QT][DK / 2], oa[QT][DK / 2];
#pragma unroll
              for (int m = 0; m < QT; ++m)
#pragma unroll
                for (int k2 = 0; k2 < DK / 2; ++k2) {
                  const int off = qix(l32, (h2 * DK / 2 + k2) * KSTEP + hh * KPL) + 32 * m * LQ;
                  qa[m][k2] = load_frag(&cQ[off]);
                  oa[m][k2] = load_frag(at(&cQ[off], kQtoDO));
                }
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int k2 = 0; k2 < DK / 2; ++k2)
#pragma unroll
                for (int m = 0; m < QT; ++m) {
                  accS[m] = E::mma(qa[m][k2], Kreg[h2 * DK / 2 + k2], accS[m]);
                  accP[m] = E::mma(oa[m][k2], Vreg[h2 * DK / 2 + k2], accP[m]);
                }
              __builtin_amdgcn_sched_barrier(0);
            }
            pf_itm = raw_item((t + 1) / RHO);
            pf_st = raw_item((t + 3) / RHO);

            PHASE(1);
            // P and dS (pairs flagged partial hide the elements outside
            // lo <= i - j <= hi), packed once to bf16 (hardware RNE
            // conversion); P stays in registers for dV, dS^T goes to LDS
            // [kv][q] for stage B
            const bool emask = MASKED && ((itm.y >> 29) & 1);
            const int mbase = (qblk - kv) * BC + rsub * BR - kvl;  // i - j = mbase + row
            T* cdSt = sdSt[b2];
            uint32_t pw[QT][8];
#pragma unroll
            for (int m = 0; m < QT; ++m)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int qb = 32 * m + 8 * gq + 4 * hh;  // 4 consecutive Q rows
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sStat[b3][qb]);
              const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sStat[b3][BR + qb]);
              float p[4], ds[4];
              // exp2(s log2(e) S - log2(e) LSE): both products rounded to
              // fp32 once (the second by the workspace prologue, once per
              // row), the first fused into the subtraction
#pragma unroll
              for (int e = 0; e < 4; ++e)
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(accS[m][4 * gq + e], a.scale_log2, -l4[e]));
              if (emask) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int dd = mbase + qb + e;
                  if (dd < a.mask_lo || dd > a.mask_hi) p[e] = 0.f;
                }
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) ds[e] = p[e] * (accP[m][4 * gq + e] - d4[e]);
              pw[m][2 * gq] = pack2_bf16(p[0], p[1]);
              pw[m][2 * gq + 1] = pack2_bf16(p[2], p[3]);
              *reinterpret_cast<uint2*>(at(cdSt, oDw[m][gq])) =
                  make_uint2(pack2_bf16(ds[0], ds[1]), pack2_bf16(ds[2], ds[3]));
            }
            PHASE(2);
            // dV += P^T dO (contraction over the sub-tile's Q rows; K slots:
            // Q rows r0 + {0..3}, r0 + 8 + {0..3}); the dO operands are read
            // before the first product
            frag bo[CS][NTD];
#pragma unroll
            for (int cc = 0; cc < CS; ++cc)
#pragma unroll
              for (int nt = 0; nt < NTD; ++nt)
                bo[cc][nt] = tr_sub(cdO, cc, nt);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cc = 0; cc < CS; ++cc) {
              const uint32_t* pc = &pw[cc / 2][4 * (cc % 2)];
              const frag pa = __builtin_bit_cast(bf16x8, make_uint4(pc[0], pc[1], pc[2], pc[3]));
#pragma unroll
              for (int nt = 0; nt < NTD; ++nt) accdV[nt] = E::mma(pa, bo[cc][nt], accdV[nt]);
            }
            __builtin_amdgcn_sched_barrier(0);
            PHASE(3);
          }
          // sub-tile t + 1 complete in LDS (every A wave its part)
          wait_staged(t + 2 < n_steps);
          __syncthreads();  // end of period t
        }
        if (a_kv >= 0) flush_dv();
      } else {
        // ---------------------------------------------------------- stage B
        float* dqa = a.dq_accum + hoff;
        T* dqo = reinterpret_cast<T*>(a.dq) + hoff;
        uint32_t* cnt_h = a.counters + (size_t)head * n_sub * NW;
        frag KT[KK];
        f32x16 accdK[NTD];
        int b_kv = -1;
        auto flush_dk = [&]() {
          T* dKg = reinterpret_cast<T*>(a.dk) + hoff;
#pragma unroll
          for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              dKg[(uint32_t)((b_kv * BC + 32 * w + crow(r, hh)) * D + nt * 32 + l32)] =
                  E::from_f32(accdK[nt][r] * a.scale);
        };
        auto counter = [&](int qtile) { return cnt_h + (size_t)qtile * NW + w; };
        const __amdgpu_buffer_rsrc_t dq_rs = make_rsrc(dqa, (uint32_t)(N * D * 4));
        const __amdgpu_buffer_rsrc_t dqo_rs = make_rsrc(dqo, (uint32_t)(N * D * 2));
        const __amdgpu_buffer_rsrc_t cnt_rs = make_rsrc(cnt_h, (uint32_t)(n_sub * NW * 4));
        // row-major chunk k (0..3) of this wave's 32 x 32 output tile (Q
        // rows 32 QW.., d columns 32 DT..): 4 consecutive columns of one
        // row; 8 lanes cover a 128-byte row
        auto chunk_off = [&](int q0, int k) {
          return (uint32_t)((q0 + 32 * QW + (lane >> 3) + 8 * k) * D + DT * 32 + 4 * (lane & 7));
        };
        auto dq_off = [&](int q0, int r) {
          if constexpr (ORDERED) return (uint32_t)((q0 + 32 * QW + l32) * D + DT * 32 + crow(r, hh));
          else return (uint32_t)((q0 + 32 * QW + crow(r, hh)) * D + DT * 32 + l32);
        };
        f32x4 lv[4];
        auto load_acc = [&](int qtile, bool live) {
          // L2-coherent loads may hit this CU's L1: drop every line read
          // before other workgroups updated it, right before the reads
          if constexpr (XL) l1_invalidate();
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t off = live ? 4 * chunk_off(qtile * BR, k) : kOutOfRange;
            lv[k] = coherent_load4<POL>(dq_rs, off);
          }
        };
        auto wait_turn = [&](int qtile, int rank) {
          if (lane == 0) {
            const uint64_t t0 = (DEBUG && a.wait_stats) ? (uint64_t)clock64() : 0;
            if (DEBUG && a.jitter_seed != 0u) {
              const uint32_t nap =
                  hash32(a.jitter_seed ^ (uint32_t)(head * 7919 + qtile * 131 + b_kv * 17 + w)) & 31u;
              for (uint32_t i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(8);
            }
            const bool poisoned = DEBUG && a.poison_q >= 0 && head == 0 && qtile == a.poison_q && rank == 0;
            uint32_t polls = 0;
            if (poisoned) polls = wait_counter(counter(qtile), 0xFFFFFFFFu, status, spin_limit);
            else if (rank > 0) polls = wait_counter(counter(qtile), (uint32_t)rank, status, spin_limit);
            if (DEBUG && a.wait_stats) {
              st_wait += (uint64_t)clock64() - t0;
              st_spun += polls > 0 ? 1u : 0u;
            }
          }
          __builtin_amdgcn_wave_barrier();
        };
        bool rel_pending = false;
        int rel_qtile = 0, rel_rank = 0;
        // Hand-off of the previous add: wait until its stores completed,
        // then store the next rank into its counter (device-coherent, every
        // lane the same word).  In the loop it is issued every period (to an
        // offset out of the counters' range, storing nothing, when no add is
        // pending) after exactly the accumulator reads (4) and the counter
        // read (1) of the period, which may stay outstanding.
        auto release_drain = [&]() {
          if (rel_pending) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            advance_counter(counter(rel_qtile), (uint32_t)rel_rank + 1u);
            rel_pending = false;
          }
        };
        auto release_in_loop = [&]() {
          __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
          const uint32_t off = rel_pending ? (uint32_t)(rel_qtile * NW + w) * 4u : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)rel_rank + 1u, cnt_rs, off, 0, kCoherent);
          rel_pending = false;
        };
        // counter value read one period earlier (none before the first
        // sub-tile: its turn is polled, so that every wait for this read
        // inside the loop sees the same operations issued after it)
        uint32_t p_seen = 0;
        __syncthreads();  // sub-tile 0 in LDS
        __syncthreads();  // period 0: stage A starts sub-tile 0

        // Periods 1 .. n_steps.  Every period issues the same sequence of
        // vector-memory operations, so that the waits the compiler places
        // for each of them count only the operations issued after it.
        for (int t = 1; t <= n_steps; ++t) {
          PHASE(6);
          {
            const int g = t - 1;
            const int b3 = g % NQB;
            const int b2 = g & 1;
            const int2 itm = uniform(raw_item(g / RHO));
            const int kv = itm.x & 0xFFFF;
            const int rank = itm.y & 0xFFFF;
            const bool last = ((itm.y >> 30) & 1) != 0;
            const int qtile = (itm.x >> 16) * RHO + (g % RHO);
            const int q0 = qtile * BR;
            if (kv != b_kv) {
              // stage A wrote this tile's K into sK one period ago
              if (b_kv >= 0) {
                flush_dk();
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): a fixed state after this rare path
              }
              b_kv = kv;
#pragma unroll
              for (int ks = 0; ks < KK; ++ks)
                KT[ks] = tr_frag(sK, qix, ks * 16 + 8 * hh, ks * 16 + 8 * hh + 4, DT * 32 + gcol, j16);
#pragma unroll
              for (int nt = 0; nt < NTD; ++nt) accdK[nt] = zero16();
            }

            PHASE(0);
            if constexpr (ORDERED) {
              // 1-2: turn check, accumulator reads for g, counter read for g + 1
              bool ready = rank == 0 || __builtin_amdgcn_readfirstlane(p_seen) == (uint32_t)rank;
              if (DEBUG && (a.jitter_seed != 0u || a.poison_q >= 0)) ready = false;
              if (DEBUG && a.wait_stats && lane == 0) st_waits += rank > 0 ? 1u : 0u;
              if (!ready) {
                release_drain();
                wait_turn(qtile, rank);
              }
              load_acc(qtile, rank > 0);
              const int gn = g + 1 < n_steps ? g + 1 : g;
              p_seen = load_relaxed_agent(counter((uniform(raw_item(gn / RHO)).x >> 16) * RHO + gn % RHO));
            }

            PHASE(1);
            // dK += dS^T Q (contraction over the sub-tile's Q rows; K slots:
            // Q rows r0 + {0..3}, r0 + 8 + {0..3}, the packed dS words stage
            // A wrote, read back from dS^T), then dQ_part = dS K for column
            // tile w (transposed when ordered).  The dK operands are all read
            // from LDS before its first product and the dQ operands while
            // the dK products run, so that the products wait for the reads'
            // latency once rather than once each.
            const T* cQ = sQ[b3];
            const T* cdSt = sdSt[b2];
            frag da[CS], bq[CS][NTD], fa[KK];
#pragma unroll
            for (int cc = 0; cc < CS; ++cc) {
              const uint2 d0 = *reinterpret_cast<const uint2*>(at(cdSt, oDr[cc][0]));
              const uint2 d1 = *reinterpret_cast<const uint2*>(at(cdSt, oDr[cc][1]));
              da[cc] = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
#pragma unroll
              for (int nt = 0; nt < NTD; ++nt)
                bq[cc][nt] = tr_sub(cQ, cc, nt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < KK; ++i) {
              accdK[i % NTD] = E::mma(da[i / NTD], bq[i / NTD][i % NTD], accdK[i % NTD]);
              fa[i] = tr_frag_at(at(cdSt, oF[i & 1][0] + 2 * i * 16 * LS), at(cdSt, oF[i & 1][1] + 2 * i * 16 * LS));
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 accQ = zero16();
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) {
              if constexpr (ORDERED) accQ = E::mma(KT[ks], fa[ks], accQ);
              else accQ = E::mma(fa[ks], KT[ks], accQ);
            }
            __builtin_amdgcn_sched_barrier(0);

            // 3: release the previous add (its stores have had the products
            // above as cover)
            PHASE(2);
            if constexpr (ORDERED) release_in_loop();
            PHASE(3);
            if (DEBUG && a.partials != nullptr) {
              float* pp = a.partials + (((size_t)head * a.n_tiles + kv) * N) * D;
#pragma unroll
              for (int r = 0; r < 16; ++r) pp[dq_off(q0, r)] = accQ[r];
            }

            PHASE(4);
            if constexpr (ORDERED) {
              // 4: the partial row-major through this wave's LDS area, added
              // to the accumulator values read at the top of the period
              float* row = sRow[w];
#pragma unroll
              for (int gq = 0; gq < 4; ++gq)
                *reinterpret_cast<f32x4*>(&row[rix(l32, 8 * gq + 4 * hh)]) =
                    f32x4{accQ[4 * gq], accQ[4 * gq + 1], accQ[4 * gq + 2], accQ[4 * gq + 3]};
              typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
              // The first contributor's accumulator values are zeros (its
              // reads were out of range) and adding them changes no value:
              // the partial is never -0, its MFMA sums starting from +0.
              if constexpr (!XL) {
                // device-coherent accumulator: all four sums first, then
                // four stores from their own registers (rewriting a store's
                // data registers waits for the store), either the
                // accumulator or (the last contributor, a uniform branch)
                // the scaled dQ in the output dtype; four stores either
                // way, so the waits after them count the same operations
                f32x4 v[4];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                  v[gq] = *reinterpret_cast<const f32x4*>(&row[rix((lane >> 3) + 8 * gq, 4 * (lane & 7))]);
                  v[gq] = lv[gq] + v[gq];
                }
                if (!last) {
                  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                  for (int gq = 0; gq < 4; ++gq) coherent_store4<POL>(dq_rs, 4 * chunk_off(q0, gq), v[gq]);
                  __builtin_amdgcn_sched_barrier(0);
                } else {
                  u32x2 pk[4];
#pragma unroll
                  for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 vs = v[gq] * a.scale;
                    pk[gq] = u32x2{pack2_bf16(vs[0], vs[1]), pack2_bf16(vs[2], vs[3])};
                  }
                  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                  for (int gq = 0; gq < 4; ++gq)
                    __builtin_amdgcn_raw_buffer_store_b64(pk[gq], dqo_rs, 2 * chunk_off(q0, gq), 0, 0);
                  __builtin_amdgcn_sched_barrier(0);
                }
              } else {
                // L2-coherent accumulator (XCD groups): both stores issued
                // every period, the one not wanted out of range (the
                // branch above measured slower here for naive and
                // descending under the causal mask)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                  f32x4 v = *reinterpret_cast<const f32x4*>(&row[rix((lane >> 3) + 8 * gq, 4 * (lane & 7))]);
                  v = lv[gq] + v;
                  const uint32_t off = chunk_off(q0, gq);
                  const f32x4 vs = v * a.scale;
                  coherent_store4<POL>(dq_rs, last ? kOutOfRange : 4 * off, v);
                  __builtin_amdgcn_raw_buffer_store_b64(
                      u32x2{pack2_bf16(vs[0], vs[1]), pack2_bf16(vs[2], vs[3])}, dqo_rs,
                      last ? 2 * off : kOutOfRange, 0, 0);
                }
              }
              if (!last) {
                rel_pending = true;
                rel_qtile = qtile;
                rel_rank = rank;
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) atomic_add_f32(&dqa[dq_off(q0, r)], accQ[r]);
            }
          }
          PHASE(5);
          __syncthreads();  // end of period t
        }
        if (b_kv >= 0) flush_dk();
        if constexpr (ORDERED) release_drain();
      }

      // next unit
      if (a.dynamic) {
        if (tid == 0)
          sUnit = (int)__hip_atomic_fetch_add(work_counter, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) + W;
        __syncthreads();
        unit = __builtin_amdgcn_readfirstlane(sUnit);
        __syncthreads();
      } else {
        unit += stride_static;
      }
    }
  };
  if (isA) run(std::true_type{}, std::false_type{});
  else if (pl.xl) run(std::false_type{}, std::true_type{});
  else run(std::false_type{}, std::false_type{});
  if (DEBUG && a.wait_stats != nullptr && lane == 0 && !isA) {
    uint64_t* st = a.wait_stats + ((size_t)blockIdx.x * NW + w) * 4;
    st[0] = st_wait;
    st[1] = st_waits;
    st[2] = st_spun;
    st[3] = (uint64_t)clock64() - st_t0;
  }
  if (DEBUG && a.phase_stats != nullptr && lane == 0) {
    uint64_t* st = a.phase_stats + ((size_t)blockIdx.x * 8 + wv) * 16;
    for (int k = 0; k < 8; ++k) st[k] = ph[k];
    st[14] = isA ? 1u : 2u;
    st[15] = (uint64_t)clock64() - ph_t0;
  }
#undef PHASE
}

template <int D, bool DEBUG>
static void* pick_pipe_d(bool masked, bool ordered) {
  if (masked)
    return ordered ? (void*)bwd_pipe_kernel<D, true, true, DEBUG> : (void*)bwd_pipe_kernel<D, true, false, DEBUG>;
  return ordered ? (void*)bwd_pipe_kernel<D, false, true, DEBUG> : (void*)bwd_pipe_kernel<D, false, false, DEBUG>;
}
template <bool DEBUG>
static void* pick_pipe(int d, bool masked, bool ordered) {
  if (d == 128) return pick_pipe_d<128, DEBUG>(masked, ordered);
  if (d == 64) return pick_pipe_d<64, DEBUG>(masked, ordered);
  return nullptr;
}

hipError_t bwd_pipe_max_coresident(int d, bool masked, bool ordered, int* blocks) {
  if (d != 128 && d != 64) return hipErrorInvalidValue;
  int per_cu = 0;
  for (int dbg = 0; dbg < 2; ++dbg) {
    void* f = dbg ? pick_pipe<true>(d, masked, ordered) : pick_pipe<false>(d, masked, ordered);
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

hipError_t launch_bwd_pipe(int d, bool masked, bool ordered, const BwdArgs& a, int grid,
                           hipStream_t stream) {
  const bool debug = a.jitter_seed != 0u || a.poison_q >= 0 || a.partials != nullptr ||
                     a.wait_stats != nullptr || a.phase_stats != nullptr;
  void* f = debug ? pick_pipe<true>(d, masked, ordered) : pick_pipe<false>(d, masked, ordered);
  if (f == nullptr) return hipErrorInvalidValue;
  BwdArgs copy = a;
  void* args[] = {&copy};
  // cooperative: every workgroup resident, which the ordered waits rely on
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(512), args, 0, stream);
}

}  // namespace dash
