// Grouped fp32 expert GEMMs (fp32 activations and weights) on gfx950 SIMT.
//
// Same two kernels as the bf16 path (SwiGLU up-projection with W1 and W3
// tiles side by side, then the W2 down-projection; open-model-atlas,
// "DeepSeek-V3.2-Exp - Mixture of experts", "All 19 steps", routed expert),
// computed with fp32 FMAs in k order.  Used by the GShard-style fp32
// workload (d=256, I=512), whose whole working set sits in the caches.
// 64 x 64 output tile per 256-thread block, 4 x 4 outputs per thread.
#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_grouped_kernel(GroupedGemmArgs args) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = SWIGLU ? 2 : 1;
  __shared__ float as[BK][BM + 4];
  __shared__ float bs[NB][BK][BN + 4];
  __shared__ int s_ts[kMaxGroups + 1];
  __shared__ int s_scratch[4];
  __shared__ int s_info[1];

  TileCoord tc;
  if (!grouped_tile_lookup<256>(args.offsets, args.n_groups, BM, BN, args.Nout, s_ts, s_scratch,
                                s_info, &tc))
    return;
  const int tid = threadIdx.x;
  const int K = args.K, Nout = args.Nout;
  const float* __restrict__ A = (const float*)args.A;

  // loader: 64 rows x 16 k per tile -> 4 elements per thread, 16 lanes per row
  const float* a_src[4];
  const float* b_src[NB][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int r = e >> 4, kk = e & 15;
    int64_t gr = tc.row0 + r;
    if (gr > tc.rend - 1) gr = tc.rend - 1;
    const int64_t src = args.row_index ? (int64_t)args.row_index[gr] : gr;
    a_src[i] = A + src * K + kk;
    const int64_t boff = ((int64_t)tc.group * Nout + tc.n0 + r) * K + kk;
    b_src[0][i] = (const float*)args.B0 + boff;
    if (SWIGLU) b_src[NB - 1][i] = (const float*)args.B1 + boff;
  }
  const int tm = tid >> 4, tn = tid & 15;
  float acc[NB][4][4];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 4, kk = e & 15;
      as[kk][r] = a_src[i][k0];
#pragma unroll
      for (int m = 0; m < NB; ++m) bs[m][kk][r] = b_src[m][i][k0];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][tm * 4 + i];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[m][j] = bs[m][kk][tn * 4 + j];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[m][j], acc[m][i][j]);
    }
    __syncthreads();
  }
  float* __restrict__ C = (float*)args.C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t grow = tc.row0 + tm * 4 + i;
    if (grow >= tc.rend) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = acc[0][i][j];
      if (SWIGLU) {
        const float g = v;
        v = g / (1.f + expf(-g)) * acc[NB - 1][i][j];
      }
      C[grow * Nout + tc.n0 + tn * 4 + j] = v;
    }
  }
}

hipError_t launch_gemm_f32_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_f32_grouped_kernel<true><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_store(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_f32_grouped_kernel<false><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
