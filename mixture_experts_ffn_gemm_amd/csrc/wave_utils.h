// Wavefront (64-lane) reduction and scan helpers for gfx950.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Butterfly reductions: at every stage lanes i and i^m combine the same two
// partials (commutatively), so every lane ends with the identical value.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = shfl_xor_u64(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o, 64);
    if (l >= o) v += w;
  }
  return v;
}

// Inclusive prefix sum over a block of NT threads (NT a multiple of 64, <= 1024).
// `scratch` holds NT/64 ints.  Returns the inclusive value; *total gets the sum.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int* scratch, int* total) {
  const int w = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane_id() == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int s = scratch[i];
    if (i < w) before += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return incl + before;
}

// float -> uint32 whose unsigned order matches the float order.
__device__ __forceinline__ uint32_t f32_to_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

}  // namespace moe
