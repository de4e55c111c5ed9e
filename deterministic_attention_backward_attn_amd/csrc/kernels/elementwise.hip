// Bandwidth-bound kernels around the backward: the row term delta, the
// workspace clear, the dQ scale-and-convert epilogue, and the ordering
// litmus.
#include "common.hpp"
#include "launch.hpp"
#include "plain_tables.hpp"

namespace dash {

// delta_i = sum_k dO_ik * O_ik (fp32).  The backward's row term: it equals
// sum_j P_ij dP_ij and needs only O and dO.  G = D / VEC lanes per row, each
// summing its VEC elements in index order, then a fixed xor-butterfly over
// the G lanes, so the result does not depend on timing.
template <typename T, int D>
__global__ void __launch_bounds__(256) preprocess_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout,
                                                         float* __restrict__ delta, long rows) {
  using E = Elt<T>;
  constexpr int VEC = E::VEC;
  constexpr int G = D / VEC;  // lanes per row (power of two, <= 64)
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gid / G;
  const int part = (int)(gid % G);
  float acc = 0.f;
  if (row < rows) {
    const uint4 ro = *reinterpret_cast<const uint4*>(o + row * D + part * VEC);
    const uint4 rd = *reinterpret_cast<const uint4*>(dout + row * D + part * VEC);
    const T* eo = reinterpret_cast<const T*>(&ro);
    const T* ed = reinterpret_cast<const T*>(&rd);
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc = __builtin_fmaf(E::to_f32(eo[j]), E::to_f32(ed[j]), acc);
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

template <typename T, int D>
static hipError_t go_pre(const void* o, const void* dout, float* delta, long rows,
                         hipStream_t s) {
  constexpr int G = D / Elt<T>::VEC;
  const long threads = rows * G;
  const long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((preprocess_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const T*>(o), reinterpret_cast<const T*>(dout), delta,
                     rows);
  return hipGetLastError();
}

hipError_t launch_preprocess(int dtype, int d, const void* o, const void* dout, float* delta,
                             long rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1 && d == 128) return go_pre<bf16_t, 128>(o, dout, delta, rows, stream);
  if (dtype == 1 && d == 64) return go_pre<bf16_t, 64>(o, dout, delta, rows, stream);
  if (dtype == 0 && d == 64) return go_pre<float, 64>(o, dout, delta, rows, stream);
  if (dtype == 0 && d == 128) return go_pre<float, 128>(o, dout, delta, rows, stream);
  return hipErrorInvalidValue;
}

// Clear n 32-bit words (a fill kernel rather than a memset node, so the
// call stays correct when a caller captures it into a graph).
__global__ void __launch_bounds__(256) zero_kernel(uint4* __restrict__ p, size_t n16,
                                                   uint32_t* __restrict__ tail, size_t n_tail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n_tail) tail[t] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n_words, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  const size_t n16 = n_words / 4;
  const size_t n_tail = n_words - n16 * 4;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(p), n16, p + n16 * 4, n_tail);
  return hipGetLastError();
}

// Backward workspace prologue: the clears and, for a plain mask, the
// schedule tables written from their closed forms (one thread per item),
// in one launch.
__global__ void __launch_bounds__(256) bwd_prologue_kernel(PrologueArgs a) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint4* c1 = reinterpret_cast<uint4*>(a.clear);
  for (size_t i = t0; i < a.clear_words / 4; i += stride) c1[i] = make_uint4(0u, 0u, 0u, 0u);
  uint4* c2 = reinterpret_cast<uint4*>(a.clear2);
  for (size_t i = t0; i < a.clear2_words / 4; i += stride) c2[i] = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = t0; i < a.lse_count; i += stride) a.lse2[i] = __fmul_rn(a.lse[i], kLog2e);
  if (a.n <= 0) return;
  const bool causal = a.causal != 0;
  for (size_t u = t0; u <= (size_t)a.units; u += stride)
    a.unit_off[u] = (int)plain::unit_off(a.n, causal, a.sched, (int)u);
  for (size_t i = t0; i < (size_t)a.items; i += stride)
    a.item[i] = plain::encode(a.n, causal, a.sched, (long)i);
}

hipError_t launch_bwd_prologue(const PrologueArgs& a, hipStream_t stream) {
  if ((a.clear_words | a.clear2_words) & 3u) return hipErrorInvalidValue;
  size_t work = a.clear_words / 4;
  if (a.clear2_words / 4 > work) work = a.clear2_words / 4;
  if ((size_t)a.items > work) work = (size_t)a.items;
  if ((size_t)a.units + 1 > work) work = (size_t)a.units + 1;
  if (a.lse_count > work) work = a.lse_count;
  size_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(bwd_prologue_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Clear whole row tiles of every head: block (t, head) zeroes the
// contiguous span of tile tiles[t] in that head, 16 bytes per store.
__global__ void __launch_bounds__(256) zero_tiles_kernel(uint4* __restrict__ base,
                                                         const int* __restrict__ tiles,
                                                         size_t tile_vec, size_t head_vec) {
  uint4* p = base + (size_t)blockIdx.y * head_vec + (size_t)tiles[blockIdx.x] * tile_vec;
  for (size_t i = threadIdx.x; i < tile_vec; i += blockDim.x) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_tiles(int dtype, void* base, const int* tiles, int count, int rows, int d,
                             int N, int BH, hipStream_t stream) {
  if (count <= 0 || BH <= 0) return hipSuccess;
  const size_t esize = dtype == 1 ? 2 : 4;
  const size_t tile_bytes = (size_t)rows * d * esize;
  if (tile_bytes % 16) return hipErrorInvalidValue;
  const size_t head_vec = (size_t)N * d * esize / 16;
  for (int h0 = 0; h0 < BH; h0 += 65535) {  // grid y is at most 65535
    const int hn = BH - h0 < 65535 ? BH - h0 : 65535;
    hipLaunchKernelGGL(zero_tiles_kernel, dim3((unsigned)count, (unsigned)hn), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(base) + (size_t)h0 * head_vec, tiles,
                       tile_bytes / 16, head_vec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// dQ = scale * dQ_accum, converted to the output dtype (RNE for bf16).
template <typename T>
__global__ void __launch_bounds__(256) dq_convert_kernel(const float4* __restrict__ acc,
                                                         T* __restrict__ dq, float scale,
                                                         size_t n4) {
  using E = Elt<T>;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = acc[i];
    dq[4 * i + 0] = E::from_f32(v.x * scale);
    dq[4 * i + 1] = E::from_f32(v.y * scale);
    dq[4 * i + 2] = E::from_f32(v.z * scale);
    dq[4 * i + 3] = E::from_f32(v.w * scale);
  }
}

hipError_t launch_dq_convert(int dtype, const float* acc, void* dq, float scale, size_t n,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t n4 = n / 4;  // n is a multiple of d >= 64
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (dtype == 1)
    hipLaunchKernelGGL(dq_convert_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(acc), reinterpret_cast<bf16_t*>(dq), scale,
                       n4);
  else
    hipLaunchKernelGGL(dq_convert_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(acc), reinterpret_cast<float*>(dq), scale,
                       n4);
  return hipGetLastError();
}

// Ordering litmus: contributor w (one wave) waits until *counter == turn[w],
// adds its row of `values` into acc with the same device-coherent
// read-modify-write, store completion wait and counter advance that the
// ordered dQ adds use, then sets the counter to turn[w] + 1.  With
// order-sensitive values any misordering or lost update changes the bits.
__global__ void __launch_bounds__(64) litmus_kernel(int len, const int* __restrict__ turn,
                                                    const float* __restrict__ values,
                                                    float* __restrict__ acc, uint32_t* counter,
                                                    uint32_t* status, uint32_t spin_limit) {
  const int w = blockIdx.x;
  const uint32_t my = (uint32_t)turn[w];
  if (threadIdx.x == 0 && my > 0) wait_counter(counter, my, status, spin_limit);
  __builtin_amdgcn_wave_barrier();
  for (int i = threadIdx.x; i < len; i += 64) {
    const float v = values[(size_t)w * len + i];
    coherent_store(&acc[i], my == 0 ? v : coherent_load(&acc[i]) + v);
  }
  wait_vm_stores();
  if (threadIdx.x == 0) advance_counter(counter, my + 1u);
}

hipError_t launch_litmus(int contributors, int len, const int* turn, const float* values,
                         float* acc, uint32_t* counter, uint32_t* status, uint32_t spin_limit,
                         hipStream_t stream) {
  void* args[] = {&len, &turn, &values, &acc, &counter, &status, &spin_limit};
  return hipLaunchCooperativeKernel((void*)litmus_kernel, dim3(contributors), dim3(64), args, 0,
                                    stream);
}

}  // namespace dash
