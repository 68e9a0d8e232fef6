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
// still spread over many CUs.  A thread issues the loads of up to 8 routed
// rows, the shared row and the residual before it adds any of them, so that
// many loads are in flight per wave; the expert rows are read once and the
// output written once, both with non-temporal accesses that do not keep them
// in the caches.
#include "moe_internal.h"

namespace moe {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4_t a = __builtin_nontemporal_load((const f32x4_t*)p);
  const f32x4_t b = __builtin_nontemporal_load((const f32x4_t*)(p + 4));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const u32x4_t a = __builtin_nontemporal_load((const u32x4_t*)p);
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
  __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]}, (f32x4_t*)p);
  __builtin_nontemporal_store(f32x4_t{v[4], v[5], v[6], v[7]}, (f32x4_t*)(p + 4));
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  u32x4_t a;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  __builtin_nontemporal_store(a, (u32x4_t*)p);
}

constexpr int kCombineBatch = 8;  // routed rows whose loads are issued together

// KC > 0: k == KC, known at compile time, so the batch has no branches for
// the compiler to sink a load into; KC == 0: any k, in batches of 8.
template <typename TA, typename TO, int KC>
__global__ __launch_bounds__(256) void combine_kernel(const TA* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate,
                                                      const TA* __restrict__ y_shared,
                                                      const TA* __restrict__ residual,
                                                      TO* __restrict__ out, int d, int k_arg) {
  const int k = KC > 0 ? KC : k_arg;
  const int64_t t = blockIdx.x;
  __shared__ int s_row[64];
  __shared__ float s_g[64];
  if (threadIdx.x < k) {
    int r = slot_row[t * k + threadIdx.x];
    MOE_DCHECK_FIX(r >= 0 && r < (int64_t)gridDim.x * k, kCheckSlot, r = 0);
    s_row[threadIdx.x] = r;
    s_g[threadIdx.x] = gate[t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * (256 * 8) + threadIdx.x * 8;
  if (c < d) {
    // every load is unconditional (a missing operand reads a row that exists
    // and is not added), so none of them waits for another
    float sh[8], res[8];
    load8<TA>((y_shared ? y_shared + t * d : y_perm) + c, sh);
    load8<TA>((residual ? residual + t * d : y_perm) + c, res);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      float v[kCombineBatch][8];
#pragma unroll
      for (int jj = 0; jj < kCombineBatch; ++jj) {
        const int j = j0 + jj < k ? j0 + jj : k - 1;
        load8<TA>(y_perm + (int64_t)s_row[j] * d + c, v[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < kCombineBatch; ++jj)
        if (j0 + jj < k) {
          const float g = s_g[j0 + jj];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[jj][i], acc[i]);
        }
    }
    // selects rather than branches, so that no load moves into a branch
    const bool has_sh = y_shared != nullptr, has_res = residual != nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = acc[i] + sh[i];
      acc[i] = has_sh ? a : acc[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = acc[i] + res[i];
      acc[i] = has_res ? a : acc[i];
    }
    store8<TO>(out + t * d + c, acc);
  }
}

template <typename TA, typename TO>
static void launch_combine_t(dim3 grid, const void* y_perm, const int32_t* slot_row,
                             const float* gate, const void* y_shared, const void* residual,
                             void* out, int d, int k, hipStream_t stream) {
  const TA* yp = (const TA*)y_perm;
  const TA* ys = (const TA*)y_shared;
  const TA* rs = (const TA*)residual;
  TO* o = (TO*)out;
  switch (k) {
#define MOE_COMBINE_K(KC)                                                                   \
  case KC:                                                                                  \
    combine_kernel<TA, TO, KC><<<grid, 256, 0, stream>>>(yp, slot_row, gate, ys, rs, o, d, k); \
    break;
    MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
    MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
#undef MOE_COMBINE_K
    default:
      combine_kernel<TA, TO, 0><<<grid, 256, 0, stream>>>(yp, slot_row, gate, ys, rs, o, d, k);
  }
}

hipError_t launch_combine(bool act_bf16, bool out_bf16, const void* y_perm,
                          const int32_t* slot_row, const float* gate, const void* y_shared,
                          const void* residual, void* out, int64_t T, int d, int k,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)cdiv(d, 256 * 8));
  if (act_bf16 && out_bf16)
    launch_combine_t<bf16_t, bf16_t>(grid, y_perm, slot_row, gate, y_shared, residual, out, d, k,
                                     stream);
  else if (act_bf16)
    launch_combine_t<bf16_t, float>(grid, y_perm, slot_row, gate, y_shared, residual, out, d, k,
                                    stream);
  else if (out_bf16)
    launch_combine_t<float, bf16_t>(grid, y_perm, slot_row, gate, y_shared, residual, out, d, k,
                                    stream);
  else
    launch_combine_t<float, float>(grid, y_perm, slot_row, gate, y_shared, residual, out, d, k,
                                   stream);
  return hipGetLastError();
}

MOE_CHECKS_READER(combine)

}  // namespace moe
