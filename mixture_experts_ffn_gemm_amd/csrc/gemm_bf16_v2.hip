// Grouped bf16 expert GEMMs on gfx950 MFMA, second generation.
//
// Expert FFN (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts",
// "All 19 steps", routed expert): g = x W1, u = x W3, h = silu(g) * u,
// E = h W2.  Up: H = silu(A W1^T) * (A W3^T) (W1 and W3 tiles of the same
// columns side by side in LDS, SwiGLU in the epilogue, A rows optionally
// gathered through row_index); down: Y = H W2^T.
//
// Workgroup: 512 threads = 8 wavefronts, 2 per SIMD.  Tile: 256 rows x 256
// MFMA output columns (up: 128 columns of g and the same 128 of u).  Wave w
// owns rows 128*(w/4) .. +128 and columns 64*(w%4) .. +64: 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, 128 fp32 accumulators.  The two waves sharing a
// SIMD own the two row halves, and a wave skips its 32-row blocks that lie
// past the expert's rows, so a tail tile costs each SIMD in proportion to
// its valid rows; while one wave waits for LDS the other issues MFMAs.
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

constexpr int NTHR = 512, NWAVE = 8;
constexpr int BM = 256, BN = 256;
constexpr int WB = 4;  // 32-row blocks per wave

template <int BK>
struct Geom {
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per row
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
  static constexpr int LOADS = STAGE_BYTES / (NTHR * 16);    // 16-byte loads per thread per stage
  static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;       // rows per 1 KiB load block
  static constexpr int ROWS_PER_256 = 256 / ROW_BYTES;       // rows per 256 B of LDS
  // A ds_read_b128 is served 16 lanes (256 B, all 64 banks) at a time; the 16
  // consecutive rows a lane group reads then land on 16 distinct bank slots.
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row / ROWS_PER_256) & (CPR - 1));
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

template <int NB>
struct Frags {
  bf16x8_t a[NB > 0 ? NB : 1];
  bf16x8_t b[2];
};

template <bool SWIGLU, int NB, int BK>
__device__ __forceinline__ void load_frags(const char* stage, int ks, int wm, int wn, int lane,
                                           Frags<NB>& f) {
  using G = Geom<BK>;
  const int l32 = lane & 31, kh = lane >> 5;
  const int chunk = 2 * ks + kh;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (SWIGLU ? j * 128 + wn * 32 : wn * 64 + j * 32) + l32;
    f.b[j] = *(const bf16x8_t*)(stage + G::A_BYTES + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = wm * 128 + i * 32 + l32;
    f.a[i] = *(const bf16x8_t*)(stage + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
  }
}

template <int NB>
__device__ __forceinline__ void mma(const Frags<NB>& f, f32x16_t (&acc)[WB][2]) {
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// The K loop of one wavefront that owns NB valid 32-row blocks (0..4).  Every
// wavefront runs the same loads and barriers whatever its NB.
//   SPREAD: the refill loads of a k-tile are issued a few at a time after each
//   k-step's MFMAs instead of all at once after the barrier, so the 8
//   wavefronts do not queue on the CU's address unit together.
template <bool SWIGLU, int NB, int BK, int NS, bool SPREAD>
__device__ __forceinline__ void kloop(int nk, const bf16_t* const (&src)[Geom<BK>::LOADS],
                                      char (*lds)[Geom<BK>::STAGE_BYTES], int wm, int wn, int wv,
                                      int lane, f32x16_t (&acc)[WB][2]) {
  using G = Geom<BK>;
  constexpr int LOADS = G::LOADS;
  constexpr int KS = BK / 16;                // k-steps per k-tile
  constexpr int LPK = LOADS / KS;            // loads issued after each k-step
  static_assert(LOADS % KS == 0, "loads per k-step");
#define V2_LOAD(kt_, st_, j_)                                                         \
  __builtin_amdgcn_global_load_lds((const void*)(src[(j_)] + (kt_) * BK),            \
                                   (lds_void*)(&lds[(st_)][(NWAVE * (j_) + wv) * 1024]), \
                                   16, 0, 0)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) V2_LOAD(s, s, j);
    }
  Frags<NB> f;
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of k-tile kt are done once at most the loads of
    // the (up to NS-2) k-tiles after it are in flight
    wait_ktile<LOADS, NS>(nk - 1 - kt);
    // every thread's loads of kt have landed, and every wavefront has
    // finished reading the stage of k-tile kt-1, which is refilled next
    __builtin_amdgcn_s_barrier();
    const bool refill = kt + NS - 1 < nk;
    const int rst = (kt + NS - 1) % NS;
    if (!SPREAD && refill) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) V2_LOAD(kt + NS - 1, rst, j);
    }
    const char* stage = lds[kt % NS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (NB > 0) {
        load_frags<SWIGLU, NB, BK>(stage, ks, wm, wn, lane, f);
        mma<NB>(f, acc);
      }
      if (SPREAD) {
        __builtin_amdgcn_sched_barrier(0);
        if (refill) {
#pragma unroll
          for (int j = ks * LPK; j < (ks + 1) * LPK; ++j) V2_LOAD(kt + NS - 1, rst, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#undef V2_LOAD
}

template <bool SWIGLU, int BK, int NS, bool SPREAD>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_v2_kernel(GroupedGemmArgs args) {
  using G = Geom<BK>;
  constexpr int LOADS = G::LOADS;
  // The tile lookup's scratch lives in the last stage, which is first
  // refilled after the first barrier of the K loop.
  __shared__ __attribute__((aligned(1024))) char lds[NS][G::STAGE_BYTES];
  int* s_ts = (int*)lds[NS - 1];
  int* s_scratch = s_ts + kMaxGroups + 8;
  int* s_info = s_scratch + NTHR / 64;

  // output columns per tile in the C matrix: up tiles cover 128 columns of H
  constexpr int CN = SWIGLU ? BN / 2 : BN;
  TileCoord tc;
  if (!grouped_tile_lookup<NTHR>(args.offsets, args.n_groups, BM, CN, args.Nout, s_ts, s_scratch,
                                 s_info, &tc))
    return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;
  const int K = args.K, Nout = args.Nout;
  const int64_t nrows64 = tc.rend - tc.row0;
  const int nrows = nrows64 < BM ? (int)nrows64 : BM;
  const int nblk = (nrows + 31) >> 5;
  int nbw = nblk - WB * wm;
  nbw = nbw < 0 ? 0 : (nbw > WB ? WB : nbw);

  // per-thread sources of the direct loads of a stage; instruction j of
  // wavefront wv fills the 1 KiB LDS block 8*j + wv
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
      if (SWIGLU) {
        Bm = (const bf16_t*)(r < 128 ? args.B0 : args.B1);
        n = tc.n0 + (r & 127);
      } else {
        Bm = (const bf16_t*)args.B0;
        n = tc.n0 + r;
      }
      if (n > Nout - 1) n = Nout - 1;
      src[j] = Bm + ((int64_t)tc.group * Nout + n) * K + G::swz(r, phys) * 8;
    }
  }

  f32x16_t acc[WB][2];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  switch (nbw) {
    case 4: kloop<SWIGLU, 4, BK, NS, SPREAD>(nk, src, lds, wm, wn, wv, lane, acc); break;
    case 3: kloop<SWIGLU, 3, BK, NS, SPREAD>(nk, src, lds, wm, wn, wv, lane, acc); break;
    case 2: kloop<SWIGLU, 2, BK, NS, SPREAD>(nk, src, lds, wm, wn, wv, lane, acc); break;
    case 1: kloop<SWIGLU, 1, BK, NS, SPREAD>(nk, src, lds, wm, wn, wv, lane, acc); break;
    default: kloop<SWIGLU, 0, BK, NS, SPREAD>(nk, src, lds, wm, wn, wv, lane, acc); break;
  }

  bf16_t* __restrict__ C = (bf16_t*)args.C;
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int i = 0; i < WB; ++i) {
    if (i >= nbw) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (row >= nrows) continue;
      bf16_t* crow = C + (tc.row0 + row) * Nout;
      if (SWIGLU) {
        const int col = tc.n0 + wn * 32 + l32;
        if (col < Nout) {
          const float g = acc[i][0][r], u = acc[i][1][r];
          crow[col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = tc.n0 + wn * 64 + j * 32 + l32;
          if (col < Nout) crow[col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// Configuration used by the library (K must be a multiple of BK).
constexpr int LIB_BK = 64, LIB_NS = 2;
constexpr bool LIB_SPREAD = false;

}  // namespace v2

hipError_t launch_gemm_bf16_v2(const GroupedGemmArgs& a, bool swiglu, hipStream_t s) {
  const int cn = swiglu ? v2::BN / 2 : v2::BN;
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, v2::BM, cn, a.Nout);
  if (grid <= 0) return hipSuccess;
  if (swiglu)
    v2::gemm_bf16_v2_kernel<true, v2::LIB_BK, v2::LIB_NS, v2::LIB_SPREAD><<<(unsigned)grid, v2::NTHR, 0, s>>>(a);
  else
    v2::gemm_bf16_v2_kernel<false, v2::LIB_BK, v2::LIB_NS, v2::LIB_SPREAD><<<(unsigned)grid, v2::NTHR, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
