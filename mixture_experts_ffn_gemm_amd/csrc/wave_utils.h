// Wavefront (64-lane) reduction and scan helpers for gfx950.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Max over the wavefront in every lane, on the VALU (DPP and lane swaps, no
// LDS round trips): partners lane^1 and lane^2 (quad permutes), then the
// mirrored lane of each 8-lane half-row and of each 16-lane row (after the
// earlier steps every group being paired holds one value, so a mirror pairs
// groups as an xor would), then the neighbouring row and the other half of
// the wavefront (v_permlane16_swap / v_permlane32_swap of a value with itself
// hand every lane its own value and its partner's).  Max is exact, so every
// lane ends with the identical value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15 - i within a row
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within a half-row

template <class T, class Step>
__device__ __forceinline__ T wave_reduce_exact(T v, Step&& step) {
  v = step.template dpp<kDppXor1>(v);
  v = step.template dpp<kDppXor2>(v);
  v = step.template dpp<kDppHalfMirror>(v);
  v = step.template dpp<kDppRowMirror>(v);
  v = step.swap16(v);
  v = step.swap32(v);
  return v;
}

struct MaxF32Step {
  template <int C>
  __device__ __forceinline__ float dpp(float v) const {
    return fmaxf(v, __uint_as_float(dpp_u32<C>(__float_as_uint(v))));
  }
  __device__ __forceinline__ float swap16(float v) const {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  __device__ __forceinline__ float swap32(float v) const {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
};

struct MaxU64Step {
  static __device__ __forceinline__ uint64_t mx(uint64_t a, uint64_t b) { return a > b ? a : b; }
  static __device__ __forceinline__ uint64_t pack(uint32_t hi, uint32_t lo) {
    return ((uint64_t)hi << 32) | lo;
  }
  template <int C>
  __device__ __forceinline__ uint64_t dpp(uint64_t v) const {
    return mx(v, pack(dpp_u32<C>((uint32_t)(v >> 32)), dpp_u32<C>((uint32_t)v)));
  }
  __device__ __forceinline__ uint64_t swap16(uint64_t v) const {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    return mx(pack(h[0], l[0]), pack(h[1], l[1]));
  }
  __device__ __forceinline__ uint64_t swap32(uint64_t v) const {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return mx(pack(h[0], l[0]), pack(h[1], l[1]));
  }
};

// Max over aligned segments of 2^STEPS lanes, in every lane of the segment:
// the first STEPS steps of the wavefront reduction above.
template <int STEPS>
__device__ __forceinline__ uint64_t segment_max_u64(uint64_t v) {
  static_assert(STEPS >= 1 && STEPS <= 6, "segments of 2 to 64 lanes");
  const MaxU64Step st;
  v = st.template dpp<kDppXor1>(v);
  if (STEPS > 1) v = st.template dpp<kDppXor2>(v);
  if (STEPS > 2) v = st.template dpp<kDppHalfMirror>(v);
  if (STEPS > 3) v = st.template dpp<kDppRowMirror>(v);
  if (STEPS > 4) v = st.swap16(v);
  if (STEPS > 5) v = st.swap32(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce_exact(v, MaxF32Step{}); }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  return wave_reduce_exact(v, MaxU64Step{});
}

// Butterfly sum: at every stage lanes i and i^m add the same two partials
// (commutatively), so every lane ends with the identical value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
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
