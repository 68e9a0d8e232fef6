// Grouped expert GEMMs with fp8 (OCP e4m3fn) block-scaled weights and bf16
// activations, for small row counts per expert (decode).
//
// The block scales follow the parameter-table note of open-model-atlas
// ("DeepSeek-V3.2-Exp - Mixture of experts": the checkpoint carries FP8 block
// scales): one fp32 scale per 128 x 128 block of the stored [Nout, K] weight
// matrix.  The expert math is the routed-expert SwiGLU of the same page.
//
// Decode is bound by streaming each selected expert's weights once, so the
// weights go straight from HBM to registers (no LDS): a tile is (expert,
// 64 output columns, up to 64 rows); each wavefront owns 16 columns over the
// whole K.  Per 64 values of K, lane (col = lane & 15, kg = lane >> 4) loads
// 16 consecutive fp8 weights of its column and feeds them to two
// v_mfma_f32_16x16x32_bf16 (8 each); the activation operand is loaded with the
// same k assignment, so the pair of MFMAs sums exactly the 64 products.  The
// partial sum of each 128-wide K block is scaled once by its block scale.
// Rows are handled in chunks of 16 (the MFMA M); chunks past the expert's row
// count are skipped.  Experts without rows own no tile and are never read.
#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 8 e4m3 codes (two dwords) -> 8 bf16, exactly (every e4m3 value is a bf16 value)
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// K loop + epilogue for NC valid 16-row chunks.  PF k-blocks (128 values of K)
// of this lane's weights are kept in flight in a register ring.
template <bool SWIGLU, int NC, int PF>
__device__ __forceinline__ void fp8_tile(const GroupedGemmArgs& args, const TileCoord& tc,
                                         int nrows) {
  constexpr int NB = SWIGLU ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int K = args.K, Nout = args.Nout, KB = K / 128;
  const int ncol0 = tc.n0 + wv * 16;

  const uint8_t* bp[NB];
  const float* sp[NB];
  {
    int n = ncol0 + col;
    if (n > Nout - 1) n = Nout - 1;
    const int64_t boff = ((int64_t)tc.group * Nout + n) * K + kg * 16;
    const int64_t soff = ((int64_t)tc.group * (Nout / 128) + (n >> 7)) * KB;
    bp[0] = (const uint8_t*)args.B0 + boff;
    sp[0] = args.S0 + soff;
    if (SWIGLU) {
      bp[NB - 1] = (const uint8_t*)args.B1 + boff;
      sp[NB - 1] = args.S1 + soff;
    }
  }
  const bf16_t* ap[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int64_t r = tc.row0 + c * 16 + col;
    if (r > tc.rend - 1) r = tc.rend - 1;
    const int64_t src = args.row_index ? (int64_t)args.row_index[r] : r;
    ap[c] = (const bf16_t*)args.A + src * K + kg * 16;
  }

  f32x4_t acc[NB][NC];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ring[PF][NB][2];
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < KB) {
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) ring[p][m][h] = *(const u32x4_t*)(bp[m] + p * 128 + h * 64);
    }

  for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int kb = kb0 + p;
      if (kb < KB) {
        u32x4_t cur[NB][2];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int h = 0; h < 2; ++h) cur[m][h] = ring[p][m][h];
        if (kb + PF < KB) {
#pragma unroll
          for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              ring[p][m][h] = *(const u32x4_t*)(bp[m] + (kb + PF) * 128 + h * 64);
        }
        float sc[NB];
#pragma unroll
        for (int m = 0; m < NB; ++m) sc[m] = sp[m][kb];
        f32x4_t tmp[NB][NC];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int c = 0; c < NC; ++c) tmp[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k0 = kb * 128 + h * 64;
          bf16x8_t blo[NB], bhi[NB];
#pragma unroll
          for (int m = 0; m < NB; ++m) {
            blo[m] = fp8x8_to_bf16(cur[m][h][0], cur[m][h][1]);
            bhi[m] = fp8x8_to_bf16(cur[m][h][2], cur[m][h][3]);
          }
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const bf16x8_t alo = *(const bf16x8_t*)(ap[c] + k0);
            const bf16x8_t ahi = *(const bf16x8_t*)(ap[c] + k0 + 8);
#pragma unroll
            for (int m = 0; m < NB; ++m) {
              tmp[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, blo[m], tmp[m][c], 0, 0, 0);
              tmp[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi[m], tmp[m][c], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[m][c] += tmp[m][c] * sc[m];
      }
    }
  }

  bf16_t* __restrict__ C = (bf16_t*)args.C;
  const int ocol = ncol0 + col;
  if (ocol >= Nout) return;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = c * 16 + 4 * kg + r;
      if (row >= nrows) continue;
      float v = acc[0][c][r];
      if (SWIGLU) v = v / (1.f + __expf(-v)) * acc[NB - 1][c][r];
      C[(tc.row0 + row) * Nout + ocol] = f32_to_bf16(v);
    }
  }
}

// The down projection's tiles are short (64 columns x K = I): a ring of 4
// k-blocks within 128 VGPRs gives four resident workgroups per CU, whose
// start-up latencies (tile lookup, row indices, activations) then overlap
// each other's weight streams.  The up projection streams two matrices over
// K = d per tile and keeps 2 workgroups per CU with a ring of 4.
template <bool SWIGLU>
__global__ __launch_bounds__(256, SWIGLU ? 1 : 4) void gemm_fp8_small_kernel(GroupedGemmArgs args) {
  constexpr int BM = 64, BN = 64;
  constexpr int PF = 4;
  __shared__ int s_ts[kMaxGroups + 1];
  __shared__ int s_scratch[4];
  __shared__ int s_info[1];
  TileCoord tc;
  if (!grouped_tile_lookup<256>(args.offsets, args.n_groups, BM, BN, args.Nout, s_ts, s_scratch,
                                s_info, &tc))
    return;
  const int64_t nrows_ = tc.rend - tc.row0;
  const int nrows = nrows_ < BM ? (int)nrows_ : BM;
  switch ((nrows + 15) >> 4) {
    case 1: fp8_tile<SWIGLU, 1, PF>(args, tc, nrows); break;
    case 2: fp8_tile<SWIGLU, 2, PF>(args, tc, nrows); break;
    case 3: fp8_tile<SWIGLU, 3, PF>(args, tc, nrows); break;
    default: fp8_tile<SWIGLU, 4, PF>(args, tc, nrows); break;
  }
}

hipError_t launch_gemm_fp8_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_fp8_small_kernel<true><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_store(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, 64, 64, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_fp8_small_kernel<false><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
