// Grouped expert GEMMs with fp8 (OCP e4m3fn) block-scaled weights and bf16
// activations, for small row counts per expert (decode).
//
// The block scales follow the parameter-table note of open-model-atlas
// ("DeepSeek-V3.2-Exp - Mixture of experts": the checkpoint carries FP8 block
// scales): one fp32 scale per 128 x 128 block of the stored [Nout, K] weight
// matrix.  The expert math is the routed-expert SwiGLU of the same page.
//
// Decode is bound by streaming each selected expert's weights once.  A tile
// is (expert, 64 output columns, up to 64 rows); each wavefront owns 16
// columns over the whole K.  Per 64 values of K, lane (col = lane & 15,
// kg = lane >> 4) holds 16 consecutive fp8 weights of its column and feeds
// them to two v_mfma_f32_16x16x32_bf16 (8 each); the activation operand uses
// the same k assignment, so the pair of MFMAs sums exactly the 64 products.
// The partial sum of each 128-wide K block is scaled once by its block scale.
// Rows are handled in chunks of 16 (the MFMA M); chunks past the expert's row
// count are skipped.  Experts without rows own no tile and are never read.
//
// Streaming.  The weights go straight from HBM into a per-lane register ring
// PF k-blocks deep, by non-temporal loads of whole 128-byte lines (a DPP lane
// rotate puts each lane's pieces in MFMA order); a k-block's weights are
// converted to bf16 before the ring slot is refilled, so the compiler never
// copies a register a load is still writing.  The activations (a few rows, L2-resident) are read once per
// workgroup, not once per wavefront: each thread loads its 16-byte pieces
// into a small register ring, writes them to one of two LDS slots a k-block
// ahead, and one barrier per k-block publishes them.  Every load is issued
// unconditionally (past the end it repeats the last k-block), so the code is
// straight-line and the compiler's wait counts keep the whole ring in flight.
// With activations read once per wavefront instead, the extra loads cost
// 25-45% of the streaming rate; with ordinary loads of half lines (the
// natural MFMA order) the weights stream about 10% slower.
#include <type_traits>

#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

namespace f8 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// the block scales are wave-uniform: constant-address loads become scalar loads
typedef __attribute__((address_space(4))) const float cfloat;

constexpr int BM = 64, BN = 64;
constexpr int NCMAX = BM / 16;          // 16-row chunks per tile
constexpr int CHUNK_BYTES = 16 * 256;   // 16 rows x 128 bf16 of one k-block
constexpr int SLOT_BYTES = NCMAX * CHUNK_BYTES;

// 8 e4m3 codes (two dwords) -> 8 bf16, exactly (every e4m3 value is a bf16 value)
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Lane L = (kg << 4) | col of an MFMA B operand needs, for the 64-wide half h
// of a k-block, the 16-byte piece 4h + kg of column col.  Load i holds, in lane
// (kg << 4) | (hh << 3) | c, piece 4hh + kg of column 8i + c; so lanes whose bit
// 3 equals h keep load h's value, and the others take load 1-h's value from
// lane L ^ 8 (a DPP rotate by 8 within the 16-lane row, written to the two
// banks of 4 lanes that have bit 3 != h).
__device__ __forceinline__ u32x4_t ring_to_mfma(const u32x4_t (&ld)[2], int h) {
  constexpr int kRowRor8 = 0x128;
  u32x4_t r;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    r[d] = h == 0 ? (uint32_t)__builtin_amdgcn_update_dpp((int)ld[0][d], (int)ld[1][d], kRowRor8, 0xf,
                                                          0xc, false)
                  : (uint32_t)__builtin_amdgcn_update_dpp((int)ld[1][d], (int)ld[0][d], kRowRor8, 0xf,
                                                          0x3, false);
  return r;
}

template <int P, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (P < N) {
    f(std::integral_constant<int, P>{});
    static_for<P + 1, N>(f);
  }
}

// k-blocks of activations held in registers ahead of their LDS write: PF
// (then the weights keep their full lead) within 16 x 16 bytes per lane.
constexpr int ra_for(int nc, int pf) {
  int r = pf;
  while (r > 1 && r * nc > 16) r /= 2;
  return r;
}

template <bool SWIGLU, int NC, int PF>
__device__ __forceinline__ void tile(const GroupedGemmArgs& args, const TileCoord& tc, int nrows,
                                     char* aring) {
  constexpr int NB = SWIGLU ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int K = args.K, Nout = args.Nout, KB = K / 128;  // KB % PF == 0
  const int ncol0 = tc.n0 + wv * 16;

  // Weights: two loads per k-block and matrix, each reading 8 whole 128-byte
  // lines (columns 8i .. 8i+7 of the wave): lane l takes column 8i + (l & 7),
  // 16-byte piece 4*((l >> 3) & 1) + (l >> 4).  Non-temporal: each line is read
  // once.  A DPP rotate by 8 lanes then gives every lane the pieces of its
  // MFMA column (see ring_to_mfma).
  const uint8_t* bp[NB];  // load i of a k-block reads 8 rows (8 * K bytes) further
  cfloat* sp[NB];
  {
    // the shared expert folded in as the last group has weights of its own
    const bool xg = args.B0x && tc.group == args.n_groups - 1;
    const int g = xg ? 0 : __builtin_amdgcn_readfirstlane(tc.group);
    const int piece = 4 * ((lane >> 3) & 1) + (lane >> 4);
    // Nout is a multiple of 128, so all 64 columns of a tile exist
    const int64_t boff = ((int64_t)g * Nout + ncol0 + (lane & 7)) * K + piece * 16;
    bp[0] = (const uint8_t*)(xg ? args.B0x : args.B0) + boff;
    if (SWIGLU) bp[NB - 1] = (const uint8_t*)(xg ? args.B1x : args.B1) + boff;
    // the wave's 16 columns lie in one 128-column scale block: scalar loads
    const int nb = __builtin_amdgcn_readfirstlane((ncol0 < Nout ? ncol0 : Nout - 1) >> 7);
    const int64_t soff = ((int64_t)g * (Nout / 128) + nb) * KB;
    sp[0] = (cfloat*)((xg ? args.S0x : args.S0) + soff);
    if (SWIGLU) sp[NB - 1] = (cfloat*)((xg ? args.S1x : args.S1) + soff);
  }
  // Activation staging: in chunk c, wave wv fills LDS rows 4wv .. 4wv+3 of
  // a slot; lane l writes row 4wv + (l >> 4), 16-byte position l & 15, with
  // the row's 16-byte piece (l & 15) ^ row (rows are 256 bytes; the XOR spreads
  // the pieces of one fragment read over all banks).  A k-block's pieces are
  // loaded into registers RA k-blocks ahead and written to LDS (two
  // slots) one k-block ahead.
  constexpr int RA = ra_for(NC, PF);
  static_assert(PF % RA == 0, "the register ring of A must repeat within PF");
  const char* asrc[NC];
  const int rl = wv * 4 + (lane >> 4);
  {
    const int piece = (lane & 15) ^ rl;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      int64_t r = tc.row0 + c * 16 + rl;
      if (r > tc.rend - 1) r = tc.rend - 1;
      int64_t src = args.row_index ? (int64_t)args.row_index[r] : r;
      MOE_DCHECK_FIX(src >= 0 && src < args.a_rows, kCheckRowIndex, src = 0);
      asrc[c] = (const char*)args.A + src * (int64_t)K * 2 + piece * 16;
    }
  }
  u32x4_t areg[RA][NC];
  auto load_a = [&](int s, int kb) {
    const int kc = kb < KB ? kb : KB - 1;
#pragma unroll
    for (int c = 0; c < NC; ++c) areg[s][c] = *(const u32x4_t*)(asrc[c] + kc * 256);
  };
  char* const wr_base = aring + rl * 256 + (lane & 15) * 16;
  auto write_a = [&](int s, int kb) {
    char* dst = wr_base + (kb & 1) * SLOT_BYTES;
#pragma unroll
    for (int c = 0; c < NC; ++c) *(u32x4_t*)(dst + c * CHUNK_BYTES) = areg[s][c];
  };

  f32x4_t acc[NB][NC];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ring[PF][NB][2];
  auto load_w = [&](int p, int kb) {
    const int kp = kb < KB ? kb : KB - 1;
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        ring[p][m][i] =
            __builtin_nontemporal_load((const u32x4_t*)(bp[m] + (int64_t)i * 8 * K + kp * 128));
  };
  // prologue: A(0) to LDS slot 0, A(1 .. RA) into the register ring, the
  // weights of k-blocks 0 .. PF-1 in flight
  load_a(0, 0);
  write_a(0, 0);
#pragma unroll
  for (int j = 1; j <= RA; ++j) load_a(j % RA, j);
#pragma unroll
  for (int p = 0; p < PF; ++p) load_w(p, p);

  // k-block kb: (1) its weights to bf16, freeing their ring slot for the
  // weights of kb+PF; (2) a barrier after this thread's LDS writes of A(kb):
  // A(kb) is complete in slot kb&1 and every wave has finished reading slot
  // (kb+1)&1 (A(kb-1)); (3) A(kb+1) from registers into that slot and A(kb+1+RA)
  // requested into the freed registers; (4) the MFMAs on A(kb) from LDS.
  // Loads past the end repeat the last k-block.
  const int lrow = col;  // MFMA A-operand row of this lane
  for (int kb0 = 0; kb0 < KB; kb0 += PF) {
    static_for<0, PF>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr int sa = (p + 1) % RA;  // register slot of A(kb+1), then of A(kb+1+RA)
      const int kb = kb0 + p;
      bf16x8_t wb[NB][2][2];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4_t w = ring_to_mfma(ring[p][m], h);
          wb[m][h][0] = fp8x8_to_bf16(w[0], w[1]);
          wb[m][h][1] = fp8x8_to_bf16(w[2], w[3]);
        }
      load_w(p, kb + PF);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's LDS writes
      __builtin_amdgcn_s_barrier();
      write_a(sa, kb + 1);
      load_a(sa, kb + 1 + RA);
      const char* slot = aring + (kb & 1) * SLOT_BYTES;
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
        const int q0 = h * 8 + kg * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const char* rowp = slot + c * CHUNK_BYTES + lrow * 256;
          const bf16x8_t alo = *(const bf16x8_t*)(rowp + ((q0 ^ lrow) << 4));
          const bf16x8_t ahi = *(const bf16x8_t*)(rowp + (((q0 + 1) ^ lrow) << 4));
#pragma unroll
          for (int m = 0; m < NB; ++m) {
            tmp[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, wb[m][h][0], tmp[m][c], 0, 0, 0);
            tmp[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, wb[m][h][1], tmp[m][c], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[m][c] += tmp[m][c] * sc[m];
    });
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

// One workgroup per tile; PF = depth of the weight ring (K / 128 must be a
// multiple of it), LB = workgroups per CU the registers are budgeted for.
template <bool SWIGLU, int PF, int LB>
__global__ __launch_bounds__(256, LB) void gemm_fp8_small_kernel(GroupedGemmArgs args) {
  // one LDS object: the two activation slots, then the tile-lookup scratch
  __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT_BYTES + (kMaxGroups + 1 + 8) * 4];
  char* aring = smem;
  int* s_ts = (int*)(smem + 2 * SLOT_BYTES);
  int* s_scratch = s_ts + kMaxGroups + 1;
  int* s_info = s_scratch + 4;
  TileCoord tc;
  if (!grouped_tile_lookup<256>(args.offsets, args.n_groups, BM, BN, args.Nout, s_ts, s_scratch,
                                s_info, &tc))
    return;
  const int64_t nrows_ = tc.rend - tc.row0;
  const int nrows = nrows_ < BM ? (int)nrows_ : BM;
  switch ((nrows + 15) >> 4) {
    case 1: tile<SWIGLU, 1, PF>(args, tc, nrows, aring); break;
    case 2: tile<SWIGLU, 2, PF>(args, tc, nrows, aring); break;
    case 3: tile<SWIGLU, 3, PF>(args, tc, nrows, aring); break;
    default: tile<SWIGLU, 4, PF>(args, tc, nrows, aring); break;
  }
}

}  // namespace f8

MOE_CHECKS_READER(gemm_fp8)

// Up: W1 and W3 streams, a ring of 4 k-blocks, two workgroups per CU.  Down:
// one stream over a short K (= I), a ring of 2 k-blocks and three workgroups
// per CU, whose start-up latencies (tile lookup, row indices) then overlap
// each other's streams.  K / 128 not a multiple of the ring: a ring of 1.
hipError_t launch_gemm_fp8_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, f8::BM, f8::BN, a.Nout);
  if (grid <= 0) return hipSuccess;
  if ((a.K / 128) % 4 == 0)
    f8::gemm_fp8_small_kernel<true, 4, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  else
    f8::gemm_fp8_small_kernel<true, 1, 2><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_store(const GroupedGemmArgs& a, hipStream_t s) {
  const int64_t grid = grouped_grid(a.max_rows, a.n_groups, f8::BM, f8::BN, a.Nout);
  if (grid <= 0) return hipSuccess;
  if ((a.K / 128) % 2 == 0)
    f8::gemm_fp8_small_kernel<false, 2, 3><<<(unsigned)grid, 256, 0, s>>>(a);
  else
    f8::gemm_fp8_small_kernel<false, 1, 3><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
