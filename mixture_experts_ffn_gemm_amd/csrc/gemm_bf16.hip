// Grouped bf16 GEMMs of the routed and shared experts on gfx950 MFMA.
//
// Expert FFN (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts",
// "All 19 steps", routed expert): g = x W1, u = x W3, a = g sigmoid(g),
// h = a * u, E = h W2.  Two kernels:
//   up:   H[r, :] = silu(A[r] W1_e) * (A[r] W3_e) for the rows r of expert e,
//         W1 and W3 tiles of the same output columns in one workgroup so the
//         SwiGLU is the epilogue; A rows may be gathered through row_index
//         (the token permutation is never materialised);
//   down: Y[r, :] = H[r] W2_e.
// Both operands are K-contiguous ([rows, K] and [Nout, K]), so LDS tiles are
// [rows][64] bf16 with a 16-byte XOR swizzle (chunk ^ (row & 7)) that keeps
// the 16-byte MFMA operand reads spread over the LDS banks.
// v_mfma_f32_32x32x16_bf16: per lane 8 bf16 of A row (lane&31), k-chunk
// (lane>>5); B likewise; the fp32 accumulator holds rows
// 8*(r/4) + 4*(lane>>5) + (r&3), column lane&31 for r in 0..15.
#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;  // bf16 elements of K per LDS stage

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.f + __expf(-g)) * u;
}

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_bf16_grouped_kernel(GroupedGemmArgs args) {
  constexpr int NB = SWIGLU ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;   // 2 x 2 wavefronts
  constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles per wavefront
  constexpr int A_CH = BM * 8 / 256;         // 16-byte chunks per thread
  constexpr int B_CH = BN * 8 / 256;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) bf16_t lds_a[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b[2][NB][BN * kBK];
  __shared__ int s_ts[kMaxGroups + 1];
  __shared__ int s_scratch[4];
  __shared__ int s_info[1];

  TileCoord tc;
  if (!grouped_tile_lookup<256>(args.offsets, args.n_groups, BM, BN, args.Nout, s_ts, s_scratch,
                                s_info, &tc))
    return;

  const int tid = threadIdx.x;
  const int K = args.K;
  const int Nout = args.Nout;
  const bf16_t* __restrict__ A = (const bf16_t*)args.A;

  // global source pointers of this thread's 16-byte chunks
  const bf16_t* a_src[A_CH];
  int a_lds[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, col = c & 7;
    int64_t gr = tc.row0 + r;
    if (gr > tc.rend - 1) gr = tc.rend - 1;
    const int64_t src = args.row_index ? (int64_t)args.row_index[gr] : gr;
    a_src[i] = A + src * K + col * 8;
    a_lds[i] = r * kBK + ((col ^ (r & 7)) << 3);
  }
  const bf16_t* b_src[NB][B_CH];
  int b_lds[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, col = c & 7;
    const int64_t off = ((int64_t)tc.group * Nout + tc.n0 + r) * K + col * 8;
    b_src[0][i] = (const bf16_t*)args.B0 + off;
    if (SWIGLU) b_src[NB - 1][i] = (const bf16_t*)args.B1 + off;
    b_lds[i] = r * kBK + ((col ^ (r & 7)) << 3);
  }

  u32x4_t ra[A_CH], rb[NB][B_CH];
#define MOE_GLOAD(kt_)                                                        \
  do {                                                                        \
    const int ko_ = (kt_) * kBK;                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) ra[i] =                  \
        *(const u32x4_t*)(a_src[i] + ko_);                                      \
    _Pragma("unroll") for (int m = 0; m < NB; ++m)                            \
        _Pragma("unroll") for (int i = 0; i < B_CH; ++i) rb[m][i] =           \
            *(const u32x4_t*)(b_src[m][i] + ko_);                               \
  } while (0)
#define MOE_LSTORE(buf_)                                                      \
  do {                                                                        \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                          \
        *(u32x4_t*)(&lds_a[(buf_)][a_lds[i]]) = ra[i];                          \
    _Pragma("unroll") for (int m = 0; m < NB; ++m)                            \
        _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                      \
            *(u32x4_t*)(&lds_b[(buf_)][m][b_lds[i]]) = rb[m][i];                \
  } while (0)

  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int l32 = lane & 31, khalf = lane >> 5;

  f32x16_t acc[NB][TM][TN];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  const int nk = K / kBK;
  MOE_GLOAD(0);
  MOE_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = 2 * ks + khalf;
      bf16x8_t af[TM], bfr[NB][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + l32;
        af[i] = *(const bf16x8_t*)(&lds_a[cur][r * kBK + ((chunk ^ (r & 7)) << 3)]);
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = wn * WN + j * 32 + l32;
          bfr[m][j] = *(const bf16x8_t*)(&lds_b[cur][m][r * kBK + ((chunk ^ (r & 7)) << 3)]);
        }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[m][i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j], acc[m][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_LSTORE(cur ^ 1);
    __syncthreads();
  }

#undef MOE_GLOAD
#undef MOE_LSTORE
  bf16_t* __restrict__ C = (bf16_t*)args.C;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      const int64_t grow = tc.row0 + row;
      if (grow >= tc.rend) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = tc.n0 + wn * WN + j * 32 + l32;
        float v = acc[0][i][j][r];
        if (SWIGLU) v = silu_mul(v, acc[NB - 1][i][j][r]);
        C[grow * Nout + col] = f32_to_bf16(v);
      }
    }
}

constexpr int kUpBM = 128, kUpBN = 128;
constexpr int kDnBM = 128, kDnBN = 128;

hipError_t launch_gemm_bf16_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, kUpBM, kUpBN, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_bf16_grouped_kernel<kUpBM, kUpBN, true><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_store(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, kDnBM, kDnBN, a.Nout);
  if (grid <= 0) return hipSuccess;
  gemm_bf16_grouped_kernel<kDnBM, kDnBN, false><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
