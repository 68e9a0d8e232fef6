// Grouped bf16 expert GEMMs on gfx950 MFMA, second generation.
//
// Expert FFN (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts",
// "All 19 steps", routed expert): g = x W1, u = x W3, h = silu(g) * u,
// E = h W2.  Up: H = silu(A W1^T) * (A W3^T) (W1 and W3 tiles of the same
// columns side by side in LDS, SwiGLU in the epilogue, A rows optionally
// gathered through row_index); down: Y = H W2^T.
//
// Workgroup tile: 256 rows x 256 MFMA output columns (up: 128 columns of g
// and the same 128 of u).  NWAVE wavefronts form a WGM x (NWAVE/WGM) grid;
// each owns (256/WGM) rows x (256*WGM/NWAVE) columns as 32x32 tiles of
// v_mfma_f32_32x32x16_bf16.  A wave skips its 32-row blocks that lie past
// the expert's rows, so a tail tile costs in proportion to its valid rows
// (the waves of one SIMD own different row ranges when NWAVE = 8).
//
// K is staged BK at a time through NS LDS stages filled by direct
// global->LDS loads (global_load_lds_dwordx4) issued NS-1 k-tiles ahead; each
// stage is waited for with an explicit vmcnt and a plain s_barrier (a fenced
// barrier would drain every load in flight).  An LDS row holds BK bf16 of one
// matrix row; its 16-byte chunks are XOR-swizzled so that the MFMA operand
// reads are free of bank conflicts.
#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

namespace v2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256;

template <int NWAVE, int WGM, int BK>
struct Geom {
  static constexpr int NTHR = NWAVE * 64;
  static constexpr int WGN = NWAVE / WGM;                     // waves along N
  static constexpr int WROWS = BM / WGM;                      // rows per wave
  static constexpr int WCOLS = BN / WGN;                      // MFMA columns per wave
  static constexpr int MB = WROWS / 32;                       // 32-row blocks per wave
  static constexpr int NT = WCOLS / 32;                       // 32-column tiles per wave
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per row
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
  static constexpr int LOADS = STAGE_BYTES / (NTHR * 16);    // 16-byte loads per thread per stage
  static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;       // rows per 1 KiB load block
  static constexpr int ROWS_PER_256 = 256 / ROW_BYTES;       // rows per 256 B of LDS
  static_assert(NT % 2 == 0, "the SwiGLU split needs an even number of column tiles");
  // A ds_read_b128 is served 16 lanes (256 B, all 64 banks) at a time; the 16
  // consecutive rows a lane group reads then land on 16 distinct bank slots.
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row / ROWS_PER_256) & (CPR - 1));
  }
  // LDS row of column tile j of wave column wn.  Up: the first NT/2 tiles are
  // W1 rows, the last NT/2 the W3 rows of the same output columns.
  template <bool SWIGLU>
  static __device__ __forceinline__ int brow(int wn, int j) {
    if (SWIGLU)
      return (j < NT / 2 ? 0 : 128) + wn * (WCOLS / 2) + (j % (NT / 2)) * 32;
    return wn * WCOLS + j * 32;
  }
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most `later` k-tiles' loads (of LOADS each) are in flight.
template <int LOADS, int L>
__device__ __forceinline__ void wait_ktile_exact(int later) {
  if (later == L)
    wait_vmcnt<L * LOADS>();
  else if constexpr (L > 0)
    wait_ktile_exact<LOADS, L - 1>(later);
}
template <int LOADS, int NS>
__device__ __forceinline__ void wait_ktile(int later) {
  if (later >= NS - 2)
    wait_vmcnt<(NS - 2) * LOADS>();
  else if constexpr (NS > 2)
    wait_ktile_exact<LOADS, NS - 3>(later);
}

// The K loop of one wavefront that owns NB valid 32-row blocks.  Every
// wavefront runs the same loads and barriers whatever its NB.
template <bool SWIGLU, int NWAVE, int WGM, int BK, int NS, int NB>
__device__ __forceinline__ void kloop(
    int nk, const bf16_t* const (&src)[Geom<NWAVE, WGM, BK>::LOADS],
    char (*lds)[Geom<NWAVE, WGM, BK>::STAGE_BYTES], int wm, int wn, int wv, int lane,
    f32x16_t (&acc)[Geom<NWAVE, WGM, BK>::MB][Geom<NWAVE, WGM, BK>::NT]) {
  using G = Geom<NWAVE, WGM, BK>;
  constexpr int LOADS = G::LOADS;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src[j] + s * BK),
                                         (lds_void*)(&lds[s][(NWAVE * j + wv) * 1024]), 16, 0, 0);
    }
  const int l32 = lane & 31, kh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of k-tile kt are done once at most the loads of
    // the (up to NS-2) k-tiles after it are in flight
    wait_ktile<LOADS, NS>(nk - 1 - kt);
    // every thread's loads of kt have landed, and every wavefront has
    // finished reading the stage of k-tile kt-1, which is refilled next
    __builtin_amdgcn_s_barrier();
    if (kt + NS - 1 < nk) {
      const int st = (kt + NS - 1) % NS;
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src[j] + (kt + NS - 1) * BK),
                                         (lds_void*)(&lds[st][(NWAVE * j + wv) * 1024]), 16, 0, 0);
    }
    const char* stage = lds[kt % NS];
    if (NB > 0) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int chunk = 2 * ks + kh;
        bf16x8_t b[G::NT], a[NB > 0 ? NB : 1];
#pragma unroll
        for (int j = 0; j < G::NT; ++j) {
          const int r = G::template brow<SWIGLU>(wn, j) + l32;
          b[j] = *(const bf16x8_t*)(stage + G::A_BYTES + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int r = wm * G::WROWS + i * 32 + l32;
          a[i] = *(const bf16x8_t*)(stage + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < G::NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
  }
}

// Dispatches the K loop on the wave's number of valid row blocks (0..MB).
template <bool SWIGLU, int NWAVE, int WGM, int BK, int NS, int NB>
__device__ __forceinline__ void kloop_dispatch(
    int nbw, int nk, const bf16_t* const (&src)[Geom<NWAVE, WGM, BK>::LOADS],
    char (*lds)[Geom<NWAVE, WGM, BK>::STAGE_BYTES], int wm, int wn, int wv, int lane,
    f32x16_t (&acc)[Geom<NWAVE, WGM, BK>::MB][Geom<NWAVE, WGM, BK>::NT]) {
  if (nbw == NB || NB == 0)
    kloop<SWIGLU, NWAVE, WGM, BK, NS, NB>(nk, src, lds, wm, wn, wv, lane, acc);
  else if constexpr (NB > 0)
    kloop_dispatch<SWIGLU, NWAVE, WGM, BK, NS, NB - 1>(nbw, nk, src, lds, wm, wn, wv, lane, acc);
}

template <bool SWIGLU, int NWAVE, int WGM, int BK, int NS>
__global__ __launch_bounds__(NWAVE * 64, 1) void gemm_bf16_v2_kernel(GroupedGemmArgs args) {
  using G = Geom<NWAVE, WGM, BK>;
  constexpr int LOADS = G::LOADS;
  // The tile lookup's scratch lives in the last stage, which is first
  // refilled after the first barrier of the K loop.
  __shared__ __attribute__((aligned(1024))) char lds[NS][G::STAGE_BYTES];
  int* s_ts = (int*)lds[NS - 1];
  int* s_scratch = s_ts + kMaxGroups + 8;
  int* s_info = s_scratch + G::NTHR / 64;

  // output columns per tile in the C matrix: up tiles cover 128 columns of H
  constexpr int CN = SWIGLU ? BN / 2 : BN;
  TileCoord tc;
  if (!grouped_tile_lookup<G::NTHR>(args.offsets, args.n_groups, BM, CN, args.Nout, s_ts,
                                    s_scratch, s_info, &tc))
    return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / G::WGN, wn = wv % G::WGN;
  const int K = args.K, Nout = args.Nout;
  const int64_t nrows64 = tc.rend - tc.row0;
  const int nrows = nrows64 < BM ? (int)nrows64 : BM;
  const int nblk = (nrows + 31) >> 5;
  int nbw = nblk - G::MB * wm;
  nbw = nbw < 0 ? 0 : (nbw > G::MB ? G::MB : nbw);

  // per-thread sources of the direct loads of a stage; instruction j of
  // wavefront wv fills the 1 KiB LDS block NWAVE*j + wv
  const bf16_t* src[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int blk = NWAVE * j + wv;
    const int rib = lane / G::CPR, phys = lane % G::CPR;
    if (blk < G::A_BYTES / 1024) {
      const int r = blk * G::ROWS_PER_KB + rib;
      int64_t gr = tc.row0 + r;
      if (gr > tc.rend - 1) gr = tc.rend - 1;
      const int64_t s = args.row_index ? (int64_t)args.row_index[gr] : gr;
      src[j] = (const bf16_t*)args.A + s * K + G::swz(r, phys) * 8;
    } else {
      const int r = (blk - G::A_BYTES / 1024) * G::ROWS_PER_KB + rib;  // 0..255
      const bf16_t* Bm;
      int n;
      const bool xg = args.B0x && tc.group == args.n_groups - 1;  // folded shared expert
      if (SWIGLU) {
        Bm = (const bf16_t*)(r < 128 ? (xg ? args.B0x : args.B0) : (xg ? args.B1x : args.B1));
        n = tc.n0 + (r & 127);
      } else {
        Bm = (const bf16_t*)(xg ? args.B0x : args.B0);
        n = tc.n0 + r;
      }
      if (n > Nout - 1) n = Nout - 1;
      src[j] = Bm + ((int64_t)(xg ? 0 : tc.group) * Nout + n) * K + G::swz(r, phys) * 8;
    }
  }

  f32x16_t acc[G::MB][G::NT];
#pragma unroll
  for (int i = 0; i < G::MB; ++i)
#pragma unroll
    for (int j = 0; j < G::NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  kloop_dispatch<SWIGLU, NWAVE, WGM, BK, NS, G::MB>(nbw, K / BK, src, lds, wm, wn, wv, lane, acc);

  bf16_t* __restrict__ C = (bf16_t*)args.C;
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int i = 0; i < G::MB; ++i) {
    if (i >= nbw) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * G::WROWS + i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (row >= nrows) continue;
      bf16_t* crow = C + (tc.row0 + row) * Nout;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < G::NT / 2; ++j) {
          const int col = tc.n0 + wn * (G::WCOLS / 2) + j * 32 + l32;
          if (col < Nout) {
            const float g = acc[i][j][r], u = acc[i][j + G::NT / 2][r];
            crow[col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < G::NT; ++j) {
          const int col = tc.n0 + wn * G::WCOLS + j * 32 + l32;
          if (col < Nout) crow[col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// Configuration used by the library (K must be a multiple of BK).
constexpr int LIB_NWAVE = 8, LIB_WGM = 2, LIB_BK = 64, LIB_NS = 2;

}  // namespace v2

hipError_t launch_gemm_bf16_v2(const GroupedGemmArgs& a, bool swiglu, hipStream_t s) {
  const int cn = swiglu ? v2::BN / 2 : v2::BN;
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, v2::BM, cn, a.Nout);
  if (grid <= 0) return hipSuccess;
  constexpr int nthr = v2::LIB_NWAVE * 64;
  if (swiglu)
    v2::gemm_bf16_v2_kernel<true, v2::LIB_NWAVE, v2::LIB_WGM, v2::LIB_BK, v2::LIB_NS>
        <<<(unsigned)grid, nthr, 0, s>>>(a);
  else
    v2::gemm_bf16_v2_kernel<false, v2::LIB_NWAVE, v2::LIB_WGM, v2::LIB_BK, v2::LIB_NS>
        <<<(unsigned)grid, nthr, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
