// Device-side building blocks shared by the attention kernels (gfx950).
//
// MFMA fragments.  All contractions use the 32x32 output MFMA:
//   bf16: v_mfma_f32_32x32x16_bf16, 8 bf16 of A and of B per lane per step
//   fp32: v_mfma_f32_32x32x2_f32,   1 float of A and of B per lane per step
// Operand A (M x K): lane l holds row l%32; operand B (K x N): lane l holds
// column l%32.  Both take their K values from the lane half h = l/32 and the
// slot s; the hardware pairs A's (h, s) with B's (h, s), so any consistent
// assignment of K indices to (h, s) is a valid contraction.
// Accumulator C (M x N): lane l holds column l%32; its register r holds row
//   crow(r, h) = 8*(r/4) + 4*h + (r%4).
// Reusing an accumulator as a K operand: the rows of a 32-row accumulator
// tile are cut into chunks of KSTEP rows; chunk c of a lane is registers
// r = KPL*c + s (s < KPL), i.e. rows crow(KPL*c + s, h).  The other operand
// is then read with exactly those row indices in its K slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int crow(int r, int h) { return ((r >> 2) << 3) + (h << 2) + (r & 3); }

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32, round to
// nearest even); bf16 -> fp32 is exact.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Element traits: storage type, MFMA fragment type and the K step.
template <typename T> struct Elt;

template <> struct Elt<float> {
  typedef float frag;
  static constexpr int KPL = 1;     // K values per lane per MFMA
  static constexpr int KSTEP = 2;   // K per MFMA
  static constexpr int VEC = 4;     // elements per 16-byte global access
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};

struct bf16_t { uint16_t bits; };

template <> struct Elt<bf16_t> {
  typedef bf16x8 frag;
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  static constexpr int VEC = 8;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(bf16_t x) { return bf16_bits_to_f32(x.bits); }
  __device__ static __forceinline__ bf16_t from_f32(float x) { return bf16_t{f32_to_bf16_bits(x)}; }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Build a bf16 fragment from 8 floats (RNE).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  uint4 u;
  u.x = pack2_bf16(v[0], v[1]);
  u.y = pack2_bf16(v[2], v[3]);
  u.z = pack2_bf16(v[4], v[5]);
  u.w = pack2_bf16(v[6], v[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// Load a K-contiguous fragment (KPL elements) from memory (LDS or global).
__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}
__device__ __forceinline__ float load_frag(const float* p) { return *p; }

// Transposing LDS read of 4 bf16: within each 16-lane group, lane j supplies
// the address of 4 consecutive elements of row (base_row + j/4), columns
// (base_col + 4*(j%4) .. +3); lane i receives column base_col + i of rows
// base_row .. base_row + 3.
__device__ __forceinline__ u16x4 lds_tr16(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(u16x4, r);
}

// Fragment whose 8 K slots are rows r0+{0..3} and r1+{0..3} of column
// c0 + (lane's index in its 16-lane half-column group) of a row-major LDS
// array; c0 already includes 16*(group%2).  `ix(row, col)` gives the element
// offset of (row, col) (padded or swizzled layouts); the 4 elements a lane
// addresses never straddle a 16-byte chunk.
template <typename IX>
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* base, IX ix, int r0, int r1, int c0,
                                          int j) {
  const u16x4 a = lds_tr16(base + ix(r0 + (j >> 2), c0 + 4 * (j & 3)));
  const u16x4 b = lds_tr16(base + ix(r1 + (j >> 2), c0 + 4 * (j & 3)));
  u16x8 u;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u[s] = a[s];
    u[s + 4] = b[s];
  }
  return __builtin_bit_cast(bf16x8, u);
}

// Bank-conflict-free layout of the bf16 row-major tiles sQ, sdO, sK (row
// stride D, no padding): the 16-byte chunk c of row r is stored at chunk
// c ^ swz(r).  The permutation keeps 16 consecutive rows of one chunk (the
// S/dP operand reads) and 4 consecutive rows of 4 consecutive chunks (the
// transposing reads) in distinct LDS banks, and every 16-lane run of the
// row-major staging writes covers whole rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return 4 * (r & 3) + ((r >> 2) & 3);
  } else {
    const int m = (r >> 1) & 7;
    return ((m & 1) << 2) | (m >> 1);
  }
}

// Device-scope counter load.
__device__ __forceinline__ uint32_t load_relaxed_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp32 add performed at the device coherence point (no return value).
__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Status word bits (workspace header).
constexpr uint32_t kStatusTimeout = 1u;

// Hand-off primitives of the ordered adds.  The shared data (the fp32 dQ
// accumulator) and the counters are only ever accessed with device-coherent
// loads and stores (the cache policy of device-scope atomics), so ordering
// needs no cache-wide write-back or invalidation: the writer waits until its
// own stores have completed before it advances the counter, and the reader
// issues its loads only after it has seen the counter value.
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-coherent accesses through a buffer resource (bounds-checked
// against num_bytes: out-of-range loads return 0, stores are dropped).  The
// cache policy is the one device-scope atomics use (sc1); 16-byte requests
// carry four times the data of per-lane dword requests.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
// Cache-policy operands: sc1 = coherent across the device (every XCD);
// sc0 = workgroup scope: a load may still be served by a line in this CU's
// L1, otherwise by the XCD's L2, so a reader of data that other CUs of the
// XCD wrote invalidates its L1 first (l1_invalidate), then reads with sc0.
constexpr int kCoherent = 16;
// Invalidate this CU's vector L1 cache (L2 untouched).
__device__ __forceinline__ void l1_invalidate() { asm volatile("buffer_inv sc0" ::: "memory"); }

// A buffer offset past every accumulator's range (the host keeps ranges
// below 2^31 bytes): loads there return 0 without a memory access.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kXcdCoherent = 1;
template <int POLICY = kCoherent>
__device__ __forceinline__ f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, POLICY));
}
template <int POLICY = kCoherent>
__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                                f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(f32x4, v), r, byte_off, 0, POLICY);
}
// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 0xFu;
}

// s_waitcnt vmcnt(0): this wave's vector memory operations have completed.
__device__ __forceinline__ void wait_vm_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void advance_counter(uint32_t* cnt, uint32_t v) {
  __hip_atomic_store(cnt, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until *cnt == target.  Called by one lane; polls with
// device-coherent loads.  Gives up after `limit` polls (or soon after another
// wait gave up) and records the time-out in *status.  Returns the number of
// failed polls.
__device__ __forceinline__ uint32_t wait_counter(const uint32_t* cnt, uint32_t target,
                                                 uint32_t* status, uint32_t limit) {
  uint32_t polls = 0;
  while (true) {
    if (load_relaxed_agent(cnt) == target) return polls;
    if ((polls & 255u) == 255u && load_relaxed_agent(status) != 0u) return polls;
    if (++polls > limit) {
      __hip_atomic_fetch_or(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return polls;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

}  // namespace dash
