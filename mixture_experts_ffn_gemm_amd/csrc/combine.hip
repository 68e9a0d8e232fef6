// Gate-weighted unpermute + shared expert + residual on gfx950.
//
// open-model-atlas ("DeepSeek-V3.2-Exp - Mixture of experts"): the routed
// output is sum_i G_i E_i and Delta = y_routed + y_shared; its forward excerpt
// accumulates the gate-weighted expert rows into an fp32 buffer.  The layer
// output adds the input (aiany.app explainer Step 7; shivam2003.com "5.6",
// Idea 2).  Each output element is summed in fp32 in a fixed order - the k
// routed terms in selection order, then y_shared, then the residual - by the
// one thread that owns it, so the result does not depend on scheduling.
// A 256-thread block covers 2048 columns of one token row (grid: tokens x
// column blocks), each thread 8 consecutive columns, so a few tokens (decode)
// still spread over many CUs.
#include "moe_internal.h"

namespace moe {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const u32x4_t a = *(const u32x4_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
  *(f32x4_t*)(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  u32x4_t a;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *(u32x4_t*)p = a;
}

template <typename TA, typename TO>
__global__ __launch_bounds__(256) void combine_kernel(const TA* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate,
                                                      const TA* __restrict__ y_shared,
                                                      const TA* __restrict__ residual,
                                                      TO* __restrict__ out, int d, int k) {
  const int64_t t = blockIdx.x;
  __shared__ int s_row[64];
  __shared__ float s_g[64];
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = slot_row[t * k + threadIdx.x];
    s_g[threadIdx.x] = gate[t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * (256 * 8) + threadIdx.x * 8;
  if (c < d) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      float v[8];
      load8<TA>(y_perm + (int64_t)s_row[j] * d + c, v);
      const float g = s_g[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    if (y_shared) {
      float v[8];
      load8<TA>(y_shared + t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (residual) {
      float v[8];
      load8<TA>(residual + t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8<TO>(out + t * d + c, acc);
  }
}

hipError_t launch_combine(bool act_bf16, bool out_bf16, const void* y_perm,
                          const int32_t* slot_row, const float* gate, const void* y_shared,
                          const void* residual, void* out, int64_t T, int d, int k,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)cdiv(d, 256 * 8));
  if (act_bf16 && out_bf16)
    combine_kernel<bf16_t, bf16_t><<<grid, 256, 0, stream>>>(
        (const bf16_t*)y_perm, slot_row, gate, (const bf16_t*)y_shared, (const bf16_t*)residual,
        (bf16_t*)out, d, k);
  else if (act_bf16)
    combine_kernel<bf16_t, float><<<grid, 256, 0, stream>>>(
        (const bf16_t*)y_perm, slot_row, gate, (const bf16_t*)y_shared, (const bf16_t*)residual,
        (float*)out, d, k);
  else if (out_bf16)
    combine_kernel<float, bf16_t><<<grid, 256, 0, stream>>>(
        (const float*)y_perm, slot_row, gate, (const float*)y_shared, (const float*)residual,
        (bf16_t*)out, d, k);
  else
    combine_kernel<float, float><<<grid, 256, 0, stream>>>(
        (const float*)y_perm, slot_row, gate, (const float*)y_shared, (const float*)residual,
        (float*)out, d, k);
  return hipGetLastError();
}

}  // namespace moe
