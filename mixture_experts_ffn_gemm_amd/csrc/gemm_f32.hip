// Grouped fp32 expert GEMMs (fp32 activations and weights) on gfx950 MFMA.
//
// The same two kernels as the bf16 path (SwiGLU up-projection with W1 and W3
// tiles side by side, then the W2 down-projection; open-model-atlas,
// "DeepSeek-V3.2-Exp - Mixture of experts", "All 19 steps", routed expert),
// for the GShard-style fp32 workload (d=256, I=512), whose whole working set
// sits in the caches.  On that workload the up and down launches together
// take 30 us, against 70 us for the fp32-FMA (SIMT) kernels they replace.
#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

// v_mfma_f32_32x32x2_f32 takes
// fp32 operands (2 k-values per instruction) and accumulates in fp32.  A
// 64 x 64 output tile per 256-thread block, one 32 x 32 MFMA tile per
// wavefront (and per matrix: W1 and W3 for the up projection); K is staged 32
// at a time through two LDS buffers, filled from registers loaded one stage
// ahead.  Lane l of an MFMA feeds row (or column) l & 31 at k-half h = l >> 5;
// instruction i of a stage takes k = 16h + i, so a lane reads 16 consecutive
// values of one LDS row.  Result element r of lane l is output row
// 8 (r / 4) + 4 (l >> 5) + (r % 4) and output column l & 31 of the wave's tile.
namespace f32m {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int BM = 64, BN = 64, BK = 32, LDSK = BK + 4;  // LDS rows padded against bank conflicts

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(GroupedGemmArgs args) {
  constexpr int NB = SWIGLU ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float as[2][BM][LDSK];
  __shared__ __attribute__((aligned(16))) float bs[2][NB][BN][LDSK];
  __shared__ int s_ts[kMaxGroups + 1];
  __shared__ int s_scratch[4];
  __shared__ int s_info[1];

  TileCoord tc;
  if (!grouped_tile_lookup<256>(args.offsets, args.n_groups, BM, BN, args.Nout, s_ts, s_scratch,
                                s_info, &tc))
    return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = args.K, Nout = args.Nout;
  const float* __restrict__ A = (const float*)args.A;

  // loader: per matrix and stage 64 rows x 32 k = 512 float4, two per thread
  const float* a_src[2];
  const float* b_src[NB][2];
  int ld_r[2], ld_c[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    ld_r[i] = q >> 3;
    ld_c[i] = (q & 7) * 4;
    int64_t gr = tc.row0 + ld_r[i];
    if (gr > tc.rend - 1) gr = tc.rend - 1;
    int64_t src = args.row_index ? (int64_t)args.row_index[gr] : gr;
    MOE_DCHECK_FIX(src >= 0 && src < args.a_rows, kCheckRowIndex, src = 0);
    a_src[i] = A + src * K + ld_c[i];
    // Nout is a multiple of 64: every weight row of the tile exists
    const int64_t boff = ((int64_t)tc.group * Nout + tc.n0 + ld_r[i]) * K + ld_c[i];
    b_src[0][i] = (const float*)args.B0 + boff;
    if (SWIGLU) b_src[NB - 1][i] = (const float*)args.B1 + boff;
  }
  f32x4_t ra[2], rb[NB][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = *(const f32x4_t*)(a_src[i] + k0);
#pragma unroll
      for (int m = 0; m < NB; ++m) rb[m][i] = *(const f32x4_t*)(b_src[m][i] + k0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(f32x4_t*)&as[buf][ld_r[i]][ld_c[i]] = ra[i];
#pragma unroll
      for (int m = 0; m < NB; ++m) *(f32x4_t*)&bs[buf][m][ld_r[i]][ld_c[i]] = rb[m][i];
    }
  };

  f32x16_t acc[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;

  const int arow = wm * 32 + (lane & 31), bcol = wn * 32 + (lane & 31), kh = (lane >> 5) * 16;
  const int nk = K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
    f32x4_t av[4], bv[NB][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = *(const f32x4_t*)&as[buf][arow][kh + 4 * q];
#pragma unroll
      for (int m = 0; m < NB; ++m) bv[m][q] = *(const f32x4_t*)&bs[buf][m][bcol][kh + 4 * q];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int m = 0; m < NB; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i >> 2][i & 3], bv[m][i >> 2][i & 3], acc[m],
                                                      0, 0, 0);
    // the other buffer was last read in the previous stage, before its barrier
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  float* __restrict__ C = (float*)args.C;
  const int ocol = tc.n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t grow = tc.row0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (grow >= tc.rend) continue;
    float v = acc[0][r];
    if (SWIGLU) v = v / (1.f + expf(-v)) * acc[NB - 1][r];
    C[grow * Nout + ocol] = v;
  }
}

}  // namespace f32m

MOE_CHECKS_READER(gemm_f32)

hipError_t launch_gemm_f32_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  f32m::gemm_f32_mfma_kernel<true><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_store(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  f32m::gemm_f32_mfma_kernel<false><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
