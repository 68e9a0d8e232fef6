// Grouped bf16 expert GEMMs on gfx950 MFMA: persistent, one wavefront per
// SIMD, with one software pipeline running across all tiles of a workgroup.
//
// Expert FFN (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts",
// "All 19 steps", routed expert): g = x W1, u = x W3, h = silu(g) * u,
// E = h W2.  Up: H = silu(A W1^T) * (A W3^T) (W1 and W3 tiles of the same
// columns side by side in LDS, SwiGLU in the epilogue, A rows optionally
// gathered through row_index); down: Y = H W2^T.
//
// Work split.  Output tiles are 256 rows x 256 MFMA columns (up: 128 columns
// of g and the same 128 of u), enumerated expert-major, then N-tile, then
// M-tile; experts with no rows own no tile and are never read.  The grid has
// one workgroup per CU.  The tile list is cut into one contiguous range per
// XCD, and the workgroups of an XCD take its tiles round-robin, so at any time
// an XCD works on consecutive tiles that share weight panels and activation
// rows through its L2.  A shared expert folded in as the last group is not
// part of that cut: each XCD takes an eighth of its M-tiles (all N-tiles of
// each) after its routed range, so that the shared expert's work, whose tiles
// all read one weight matrix, is spread over the eight XCDs instead of
// landing on the last one.  Every workgroup rebuilds the per-expert tile
// prefix from the device offsets in LDS; the host never waits for the counts.
//
// Workgroup: 256 threads = 4 wavefronts, one per SIMD.  With bf16 weights
// wave w owns the 32-row blocks w/2, w/2+2, .. and columns 128*(w%2) .. +128
// of the tile, as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16; with fp8 weights
// it owns all eight row blocks and columns 64w .. +64 (8 x 2 tiles).  The
// weight fragment is the first MFMA operand, so each lane accumulates 4 runs
// of 4 consecutive output columns of one row (256 fp32 accumulators in the
// AGPRs).  A lane pair (l, l+32) trades halves with v_permlane32_swap in the
// epilogue and each lane stores 16 bytes.
//
// Every tile does all of its MFMAs, also past an expert's last row (those
// rows are not stored): tiles of equal cost keep the workgroups of an XCD in
// step, so the panels they share are still in L2 when each of them reads
// them.  Skipping the MFMAs of a partly filled tile made such tiles finish
// early, the workgroups drifted apart and the routed up projection of the
// V3-shaped layer read 37 GB past L2 instead of 21 GB and ran 10-19% slower.
// The rows past the end read rows of zeros when the caller provides them
// (zero_row: kZeroRows rows of K), else repeat the last row: the chip runs
// these GEMMs at a clock set by power, and MFMAs on zero operands draw less
// of it (with all activations zero the routed up projection runs 18% faster).
// Row r of a tile reads zero row r % kZeroRows, so that the padding loads of
// all workgroups spread over the L2 channels instead of meeting on one line.
//
// Pipeline.  K is staged BK at a time through NS LDS stages by direct
// global->LDS loads (global_load_lds_dwordx4).  A "step" is one BK slice of one
// tile; the steps of all tiles of the workgroup form one sequence, and the
// loads of step q+NS-1 are issued during step q, one or two at a time between
// groups of four MFMAs, so the texture path sees an even stream instead of a
// burst.  The fragments of the next k-step are read from LDS while the MFMAs of
// the current one run.  One barrier per step, between the two halves of the
// last k-step's MFMAs.  The gathered row indices of the tile after next are
// fetched into LDS by a direct load too, so no load result is ever waited for
// in registers.  LDS rows hold BK bf16 of one matrix row; their 16-byte chunks
// are XOR-swizzled so the fragment reads are free of bank conflicts.
//
// fp8 weights (W8).  The weights may be OCP e4m3fn codes with one fp32 scale
// per 128 x 128 block (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of
// experts", the parameter table's note on FP8 block scales).  Their LDS rows
// then hold 32 codes (two 16-byte halves, the halves of rows 8..15 of every
// 16 swapped so 16 lanes' reads cover all banks); a lane reads its 16 codes for
// both k-steps of a step at once and dequantizes them to bf16 as
// bf16(code * scale) (code to fp32 exactly, one fp32 multiply, round to nearest
// even) just before its MFMAs.  The k-values a lane group feeds to one MFMA
// are then 16g + 8ks + 0..7 rather than 8(2ks + g) + 0..7; the activation
// fragments follow the same assignment, so every MFMA still pairs equal k.
// A step's tile is 16 KiB of activations and 8 KiB of codes.  Each wave
// owns 64 columns of all 256 rows, so every code is dequantized once per
// workgroup (64 VALU instructions per wave and step; with the bf16 layout of
// 128 x 128 per wave two waves dequantized each column, twice the VALU work,
// and the routed up + down GEMMs of the V3-shaped prefill took 13.22 ms
// against 12.91 ms).  The dequantization is issued in between the MFMAs of
// its unit, a share after each MFMA: a wavefront issues in order, so a run
// of VALU instructions after a group of MFMAs left the matrix core idle once
// the group's last MFMA had finished (with the bf16 layout: 14.7 ms with the
// VALU after each group, 13.8 ms interleaved, 13.2 ms interleaved and with
// the barrier one group earlier; the same schedule for the bf16 path's
// memory instructions was 8% slower).
#include <atomic>

#include "grouped_sched.h"
#include "moe_internal.h"

namespace moe {

namespace gp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
// block scales are wave-uniform: constant-address loads become scalar loads
typedef __attribute__((address_space(4))) const float cfloat;

constexpr int BM = 256, BN = 256, NTHR = 256, NWAVE = 4;

// Wave layout in the 256 x 256 tile, as MB 32-row blocks x NT 32-column
// tiles of MFMAs per wave (256 fp32 accumulators either way).  bf16 weights:
// wave w owns row blocks w/2, w/2+2, .. and columns 128*(w%2) .. +128.  fp8
// weights: wave w owns all eight row blocks and columns 64w .. +64, so that
// each weight code is dequantized by one wave instead of two (half the VALU
// work per step, for twice the activation fragment reads).
template <bool W8>
struct Lay {
  static constexpr int MB = W8 ? 8 : 4, NT = W8 ? 2 : 4;
  // row block of the wave's i-th row of MFMAs
  static __device__ __forceinline__ int rblk(int i, int wv) { return W8 ? i : 2 * i + (wv >> 1); }
  // the wave's column slot: 32*NT columns from 32*NT*wcol(wv) on
  static __device__ __forceinline__ int wcol(int wv) { return W8 ? wv : (wv & 1); }
};

template <int BK, bool W8>
struct Geo {
  static_assert(!W8 || BK == 32, "fp8 rows are two 16-byte halves");
  static constexpr int ROW_BYTES = BK * 2;                // activation LDS row
  static constexpr int B_ROW_BYTES = W8 ? BK : BK * 2;    // weight LDS row
  static constexpr int CPR = BK / 8;                      // 16-byte chunks per activation row
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int B_BYTES = BN * B_ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LOADS = STAGE_BYTES / (NTHR * 16); // direct loads per thread per step
  static constexpr int A_LOADS = A_BYTES / (NTHR * 16);
  static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
  static constexpr int B_ROWS_PER_KB = 1024 / B_ROW_BYTES;
  static constexpr int ROWS_PER_256 = 256 / ROW_BYTES;
  static constexpr int KS = BK / 16;                      // k-steps per step
  static constexpr int B_STEP = BK * (W8 ? 1 : 2);        // weight bytes per row per step
  // A ds_read_b128 is served 16 lanes (256 B, all 64 banks) at a time; the
  // 16 consecutive rows a lane group reads then land on 16 distinct slots.
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row / ROWS_PER_256) & (CPR - 1));
  }
  // fp8 weight rows: 16-byte half h of row r sits at position h ^ ((r >> 3) & 1)
  static __device__ __forceinline__ int swz8(int row, int half) { return half ^ ((row >> 3) & 1); }
  // activation chunk of lane group g (lane >> 5) in k-step ks
  static __device__ __forceinline__ int achunk(int ks, int g) { return W8 ? 2 * g + ks : 2 * ks + g; }
};

// LDS row of column tile j of the wave in column slot wc.  Up: the first
// half of the tiles are W1 rows, the second half the W3 rows of the same
// output columns.
template <bool SWIGLU, bool W8>
__device__ __forceinline__ int brow(int wc, int j) {
  constexpr int NT = Lay<W8>::NT, H = NT / 2;
  if (SWIGLU) return (j < H ? 0 : 128) + wc * 32 * H + (j % H) * 32;
  return wc * 32 * NT + j * 32;
}

// s_waitcnt on the vector-memory counter (gfx9 encoding), and on every LDS
// access of this wavefront too.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

template <bool W8>
struct Frags {
  bf16x8_t a[Lay<W8>::MB], b[Lay<W8>::NT];
};

// Activation fragments of rows lo .. lo+n-1 of the wave's MFMA rows.
template <int BK, bool W8>
__device__ __forceinline__ void read_a(const char* stage, int ks, int wv, int lane, Frags<W8>& f,
                                       int lo = 0, int n = Lay<W8>::MB) {
  using G = Geo<BK, W8>;
  const int l32 = lane & 31, chunk = G::achunk(ks, lane >> 5);
#pragma unroll
  for (int i = 0; i < Lay<W8>::MB; ++i) {
    if (i < lo || i >= lo + n) continue;
    const int r = Lay<W8>::rblk(i, wv) * 32 + l32;
    f.a[i] = *(const bf16x8_t*)(stage + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
  }
}

// bf16 weight fragments of the wave's column tiles.
template <int BK, bool SWIGLU>
__device__ __forceinline__ void read_b(const char* stage, int ks, int wv, int lane,
                                       Frags<false>& f) {
  using G = Geo<BK, false>;
  const int l32 = lane & 31, chunk = G::achunk(ks, lane >> 5);
#pragma unroll
  for (int j = 0; j < Lay<false>::NT; ++j) {
    const int r = brow<SWIGLU, false>(Lay<false>::wcol(wv), j) + l32;
    f.b[j] = *(const bf16x8_t*)(stage + G::A_BYTES + r * G::ROW_BYTES + (G::swz(r, chunk) << 4));
  }
}

// fp8 weights: the two block scales of this wave's columns in one step (W1
// and W3 for the up projection; the down projection uses s0 for all).
struct StepScale {
  float s0, s1;
};

// e4m3 codes k0 .. k0+N-1 of the 8 in (w0, w1) -> bf16(code * s) into
// d[k0 ..], round to nearest even
template <int K0, int N>
__device__ __forceinline__ void dequant(uint32_t w0, uint32_t w1, float s, bf16x8_t& d) {
#pragma unroll
  for (int p = K0 / 2; p < (K0 + N) / 2; ++p) {
    const uint32_t w = p < 2 ? w0 : w1;
    const f32x2_t v = (p & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true)
                              : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    d[2 * p] = (__bf16)(v[0] * s);
    d[2 * p + 1] = (__bf16)(v[1] * s);
  }
}

// fp8 weights: the lane's 16 codes of each column tile for both k-steps of a
// step (the first 8 for k-step 0, the last 8 for k-step 1).
template <int BK, bool SWIGLU>
__device__ __forceinline__ void read_w8_raw(const char* stage, int wv, int lane,
                                            u32x4_t (&raw)[Lay<true>::NT]) {
  using G = Geo<BK, true>;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int j = 0; j < Lay<true>::NT; ++j) {
    const int r = brow<SWIGLU, true>(Lay<true>::wcol(wv), j) + l32;
    raw[j] = *(const u32x4_t*)(stage + G::A_BYTES + r * G::B_ROW_BYTES + (G::swz8(r, g) << 4));
  }
}
// codes K0 .. K0+N-1 of column tile j of k-step ks, dequantized (the W3
// tiles take s1 in the up projection)
template <bool SWIGLU, int K0 = 0, int N = 8>
__device__ __forceinline__ void dequant_tile(const u32x4_t (&raw)[Lay<true>::NT], int j, int ks,
                                             StepScale sc, Frags<true>& f) {
  dequant<K0, N>(raw[j][2 * ks], raw[j][2 * ks + 1],
                 SWIGLU && j >= Lay<true>::NT / 2 ? sc.s1 : sc.s0, f.b[j]);
}

// The MFMAs of the wave's row i of one k-step.
template <bool W8>
__device__ __forceinline__ void mfma_row(int i, const Frags<W8>& f,
                                         f32x16_t (&acc)[Lay<W8>::MB][Lay<W8>::NT]) {
#pragma unroll
  for (int j = 0; j < Lay<W8>::NT; ++j)
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Per-workgroup tile table in LDS.
struct TileTab {
  int ts[kMaxGroups + 1];   // exclusive prefix of M-tiles per group
  int off[kMaxGroups + 1];  // row offsets of the groups
  int scan[NTHR / 64];
  int ri[2][BM];            // gathered row indices of upcoming tiles
};

struct Tile {
  int g, n0;
  int64_t row0, rend;
};

__device__ __forceinline__ Tile decode_tile(const TileTab& tt, int n_groups, int ntn, int CN,
                                            int L) {
  // the group g with ts[g]*ntn <= L < ts[g+1]*ntn (ts[0] = 0, ts[n] * ntn > L)
  int lo = 0, hi = n_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tt.ts[mid] * ntn <= L) lo = mid;
    else hi = mid;
  }
  const int tiles_g = tt.ts[lo + 1] - tt.ts[lo];
  const int rem = L - tt.ts[lo] * ntn;
  Tile t;
  t.g = lo;
  t.row0 = (int64_t)tt.off[lo] + (int64_t)(rem % tiles_g) * BM;
  t.rend = tt.off[lo + 1];
  t.n0 = (rem / tiles_g) * CN;
  return t;
}

// The issue side of the pipeline: which step's slice the next direct loads
// fetch, and their sources in the current tile: for activation rows a
// per-lane address (a row past the tile's last reads the zero row), for
// weight rows a wave-uniform base and a 32-bit per-lane byte offset.
template <int BK, bool SWIGLU, bool W8>
struct Issuer {
  using G = Geo<BK, W8>;
  const char* arow[G::A_LOADS];
  const char* base[G::LOADS];
  unsigned off[G::LOADS];
  int it, kt;  // tile index within this workgroup's list, step within the tile

  __device__ __forceinline__ void build(const GroupedGemmArgs& a, const TileTab& tt,
                                        const Tile& t, int wv, int lane) {
    const int rib = lane / G::CPR, phys = lane % G::CPR;
    const int64_t rowb = (int64_t)a.K * 2;           // bytes per activation row
    const int64_t browb = (int64_t)a.K * (W8 ? 1 : 2);  // bytes per weight row
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
      const int blk = NWAVE * j + wv;
      if (j < G::A_LOADS) {
        const int r = blk * G::ROWS_PER_KB + rib;
        int64_t row;
        if (a.row_index) {
          row = tt.ri[it & 1][r];
        } else {
          row = t.row0 + r;
          if (row > t.rend - 1) row = t.rend - 1;
        }
        MOE_DCHECK_FIX(row >= 0 && row < a.a_rows, kCheckRowIndex, row = 0);
        const bool pad = a.zero_row && t.row0 + r >= t.rend;
        arow[j] = (pad ? (const char*)a.zero_row + (r % kZeroRows) * rowb
                       : (const char*)a.A + row * rowb) +
                  (G::swz(r, phys) << 4);
      } else {
        // first LDS row of the block (0..255), this lane's row in it, and the
        // 16-byte piece of the row's step slice that goes to this lane's slot
        const int r0 = (blk - G::A_BYTES / 1024) * G::B_ROWS_PER_KB;
        const int rl = W8 ? lane >> 1 : rib;
        const int piece = W8 ? G::swz8(r0 + rl, lane & 1) : G::swz(r0 + rl, phys);
        const bool w3 = SWIGLU && r0 >= 128;
        int n = t.n0 + (SWIGLU ? (r0 & 127) : r0);
        int lim = a.Nout - 1 - n;  // rows past the last weight row repeat it
        if (lim < 0) {
          n = a.Nout - 1;
          lim = 0;
        }
        if (a.B0x && t.g == a.n_groups - 1)  // the folded shared expert
          base[j] = (const char*)(w3 ? a.B1x : a.B0x) + (int64_t)n * browb;
        else
          base[j] = (const char*)(w3 ? a.B1 : a.B0) + ((int64_t)t.g * a.Nout + n) * browb;
        off[j] = (unsigned)((rl < lim ? rl : lim) * browb) + (unsigned)(piece << 4);
      }
    }
  }

  // Direct load j of the current step into `stage`.
  __device__ __forceinline__ void load(int j, char* stage, int wv) const {
    const char* src = j < G::A_LOADS ? arow[j] + kt * (BK * 2) : base[j] + kt * G::B_STEP + off[j];
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (lds_void*)(stage + (NWAVE * j + wv) * 1024), 16, 0, 0);
  }
};

// fp8 weights: where this wave's block scales of a tile start (one 128-row
// block of W1 and of W3 for the up projection, of W2 for the down projection).
struct TileScale {
  cfloat *p0, *p1;
};
template <bool SWIGLU>
__device__ __forceinline__ TileScale tile_scale(const GroupedGemmArgs& a, const Tile& t, int wv) {
  const int KB = a.K / 128, NBL = a.Nout / 128;
  // the down projection's wave columns 32*NT*wcol .. +32*NT lie in one block
  int nb = (t.n0 >> 7) + (SWIGLU ? 0 : (32 * Lay<true>::NT * Lay<true>::wcol(wv)) >> 7);
  if (nb > NBL - 1) nb = NBL - 1;  // columns past Nout: computed, never stored
  nb = __builtin_amdgcn_readfirstlane(nb);
  const int g = __builtin_amdgcn_readfirstlane(t.g);
  const bool xg = a.B0x && g == a.n_groups - 1;
  const int64_t o = ((xg ? 0 : (int64_t)g * NBL) + nb) * KB;
  TileScale ts;
  ts.p0 = (cfloat*)((xg ? a.S0x : a.S0) + o);
  ts.p1 = SWIGLU ? (cfloat*)((xg ? a.S1x : a.S1) + o) : ts.p0;
  return ts;
}
// the scales of step kt (32 values of K; 4 steps per 128-wide block)
__device__ __forceinline__ StepScale step_scale(const TileScale& ts, int kt) {
  return StepScale{ts.p0[kt >> 2], ts.p1[kt >> 2]};
}

// The gathered row indices of tile `t` into ri[b]: wave wv fetches 64 of them.
__device__ __forceinline__ void fetch_rows(const GroupedGemmArgs& a, TileTab& tt, int b,
                                           const Tile& t, int wv, int lane) {
  int64_t gr = t.row0 + wv * 64 + lane;
  if (gr > t.rend - 1) gr = t.rend - 1;
  __builtin_amdgcn_global_load_lds((const void*)(a.row_index + gr),
                                   (lds_void*)(&tt.ri[b][wv * 64]), 4, 0, 0);
}

// This workgroup's share of its XCD's tile list.  The list holds a range of
// the tiles of the expert groups (expert-major, then N-tile, then M-tile:
// rcnt tiles from global tile rlo on), followed, when the shared expert is
// folded in as the last group, by this XCD's eighth of that group's M-tiles
// (scnt tiles from M-tile smlo on, M-tile-major: the XCD's rows meet all
// N-tiles while they are in L2).  Workgroup `slot` of the XCD takes list
// entries slot, slot + nslot, ...
struct Sched {
  int n_groups, ntn, CN, nslot, slot, ntile;
  int rlo, rcnt, smlo, scnt;
};

__device__ __forceinline__ Tile sched_tile(const TileTab& tt, const Sched& sc, int i) {
  const int j = sc.slot + i * sc.nslot;
  if (j < sc.rcnt) return decode_tile(tt, sc.n_groups, sc.ntn, sc.CN, sc.rlo + j);
  const int q = j - sc.rcnt, g = sc.n_groups - 1;
  Tile t;
  t.g = g;
  t.row0 = (int64_t)tt.off[g] + (int64_t)(sc.smlo + q / sc.ntn) * BM;
  t.rend = tt.off[g + 1];
  t.n0 = (q % sc.ntn) * sc.CN;
  return t;
}

// Advances the issuer past the step it has just loaded; on entering a new
// tile, rebuilds the sources (from row indices fetched a tile earlier) and
// fetches the row indices of the tile after it.  Past the last tile the last
// step is loaded again, into stages that are never read.
template <int BK, bool SWIGLU, bool W8>
__device__ __forceinline__ void advance(Issuer<BK, SWIGLU, W8>& is, const GroupedGemmArgs& a,
                                        TileTab& tt, const Sched& sc, int nk, int wv, int lane) {
  if (++is.kt < nk) return;
  if (is.it + 1 >= sc.ntile) {
    is.kt = nk - 1;
    return;
  }
  ++is.it;
  is.kt = 0;
  const Tile t = sched_tile(tt, sc, is.it);
  is.build(a, tt, t, wv, lane);
  if (a.row_index && is.it + 1 < sc.ntile)
    fetch_rows(a, tt, (is.it + 1) & 1,
               sched_tile(tt, sc, is.it + 1), wv, lane);
}

// Stores the finished tile: SwiGLU (up) or plain (down), bf16, 16 bytes per
// lane.  Lane l holds output row l&31 of each 32-row block and columns
// 8*q + 4*(l>>5) + 0..3 (q = 0..3) of each 32-column tile; after the swap
// with lane l^32, lane l holds columns 16*p + 8*(l>>5) + 0..7 (p = 0, 1).
template <bool SWIGLU, bool W8>
__device__ __forceinline__ void store_tile(const GroupedGemmArgs& a, const Tile& t, int wv,
                                           int lane,
                                           f32x16_t (&acc)[Lay<W8>::MB][Lay<W8>::NT]) {
  constexpr int MB = Lay<W8>::MB, NT = Lay<W8>::NT, H = NT / 2;
  constexpr int NJ = SWIGLU ? H : NT;
  constexpr int WCOLS = 32 * NJ;  // output columns per wave
  bf16_t* __restrict__ C = (bf16_t*)a.C;
  const int hi = lane >> 5;
  const int64_t nrows = t.rend - t.row0;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = Lay<W8>::rblk(i, wv) * 32 + (lane & 31);
    const bool row_ok = m < nrows;
    bf16_t* crow = C + (t.row0 + m) * a.Nout;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // keep the accumulators in the AGPRs until their tile is stored (else
      // the compiler copies all of them to VGPRs at once, and spills)
      asm volatile("" : "+a"(acc[i][j]));
      if (SWIGLU) asm volatile("" : "+a"(acc[i][j + H]));
      unsigned p[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v0, v1;
          if (SWIGLU) {
            const float g0 = acc[i][j][4 * q + 2 * h], u0 = acc[i][j + H][4 * q + 2 * h];
            const float g1 = acc[i][j][4 * q + 2 * h + 1], u1 = acc[i][j + H][4 * q + 2 * h + 1];
            v0 = g0 * __builtin_amdgcn_rcpf(1.f + __expf(-g0)) * u0;
            v1 = g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * u1;
          } else {
            v0 = acc[i][j][4 * q + 2 * h];
            v1 = acc[i][j][4 * q + 2 * h + 1];
          }
          // v_cvt_pk_bf16_f32: round to nearest even
          const bf16x2_t pk = {(__bf16)v0, (__bf16)v1};
          p[q][h] = __builtin_bit_cast(unsigned, pk);
        }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        // lanes 0-31 give their run 2pp+1 to lanes 32-63 and take those
        // lanes' run 2pp
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto r = __builtin_amdgcn_permlane32_swap(p[2 * pp][h], p[2 * pp + 1][h], false,
                                                          false);
          p[2 * pp][h] = r[0];
          p[2 * pp + 1][h] = r[1];
        }
        const int col = t.n0 + Lay<W8>::wcol(wv) * WCOLS + j * 32 + 16 * pp + 8 * hi;
        if (row_ok && col < a.Nout) {
          const u32x4_t v = {p[2 * pp][0], p[2 * pp][1], p[2 * pp + 1][0], p[2 * pp + 1][1]};
          *(u32x4_t*)(crow + col) = v;
        }
      }
      // one 32x32 tile at a time: keeps the accumulators in the AGPRs
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The four MFMAs of unit q (0..3) of one k-step: row q of the bf16 layout,
// rows 2q and 2q+1 of the fp8 one.
template <bool W8>
__device__ __forceinline__ void mfma_unit(int q, const Frags<W8>& f,
                                          f32x16_t (&acc)[Lay<W8>::MB][Lay<W8>::NT]) {
  if constexpr (W8) {
    mfma_row<true>(2 * q, f, acc);
    mfma_row<true>(2 * q + 1, f, acc);
  } else {
    mfma_row<false>(q, f, acc);
  }
}

// The steps of one tile.  Each k-step is four units of four MFMAs.  Step g of
// the sequence reads stage g % NS; during it the loads of step g+NS-1 go into
// stage (g-1) % NS, which every wave finished reading before barrier B(g).
// B(g+1) follows this thread's wait for its loads of step g+1 and for all its
// LDS reads: after it step g+1 has landed for every thread.  fp8 weights: `ss`
// holds the block scales of the current step on entry and of the next one
// (the next tile's first, `tsn`, after the last step) on return.
template <int BK, int NS, bool SWIGLU, bool W8>
__device__ __forceinline__ void run_tile(int& g, int nk, Issuer<BK, SWIGLU, W8>& is,
                                         const GroupedGemmArgs& a, TileTab& tt, const Sched& sc,
                                         char (*st)[Geo<BK, W8>::STAGE_BYTES], int wv, int lane,
                                         Frags<W8> (&f)[2],
                                         f32x16_t (&acc)[Lay<W8>::MB][Lay<W8>::NT],
                                         const TileScale& tsc, const TileScale& tsn, StepScale& ss,
                                         u32x4_t (&raw)[Lay<true>::NT]) {
  using G = Geo<BK, W8>;
  constexpr int KS = G::KS, LOADS = G::LOADS;
  // unit of the last k-step before which B(g+1) sits: fp8 weights one unit
  // earlier, so that the next step's codes, read right after it, have landed
  // before the two units that dequantize them.  The loads of a step are
  // spread over the GROUPS units before it.
  constexpr int BARI = W8 ? 1 : 2;
  constexpr int GROUPS = 4 * (KS - 1) + BARI;
  // The activation fragments of a step's second k-step are read after its
  // first S1 units, R1 rows after each (fp8 weights: eight reads in two
  // halves measured 3% faster than at once; bf16 weights, and splits into
  // four, gained nothing); those of the next step's first k-step after B(g+1).
  constexpr int MB = Lay<W8>::MB, S1 = W8 ? 2 : 1, R1 = MB / S1;
  // fp8 weights: the next step's first k-step is dequantized in the NU units
  // after the unit that B(g+1) precedes, TPU column tiles in each
  constexpr int NU = 2, TPU = Lay<true>::NT / NU;
  static_assert(BARI + NU <= 3 || !W8, "dequantization units after B(g+1)");
  static_assert(Lay<true>::NT == 2, "first k-step: half a column tile per unit");
  for (int kt = 0; kt < nk; ++kt, ++g) {
    const char* cur = st[g % NS];
    char* dst = st[(g + NS - 1) % NS];
    StepScale ss_next{0.f, 0.f};
    if constexpr (W8) {
      // scalar loads, early: the scales of the step whose fragments the
      // barrier of this step reads
      const bool last = kt + 1 >= nk;
      const TileScale& tn = last ? tsn : tsc;
      ss_next = step_scale(tn, last ? 0 : kt + 1);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Frags<W8>& fc = f[s & 1];
      Frags<W8>& fn = f[(s + 1) & 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int grp = 4 * s + q;
        if (s == KS - 1 && q == BARI) {
          // B(g+1), then the fragments of the next step's first k-step (fp8
          // weights: its codes, dequantized after this and the next unit)
          wait_vm_lgkm<(NS - 2) * LOADS>();
          __builtin_amdgcn_s_barrier();
          if constexpr (W8) read_w8_raw<BK, SWIGLU>(st[(g + 1) % NS], wv, lane, raw);
          else read_b<BK, SWIGLU>(st[(g + 1) % NS], 0, wv, lane, fn);
          read_a<BK, W8>(st[(g + 1) % NS], 0, wv, lane, fn);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_unit<W8>(q, fc, acc);
        if constexpr (W8) {
          // dequantization issued between the unit's four MFMAs.  First
          // k-step: half a column tile of the second k-step per unit (8 VALU
          // instructions); last k-step: the next step's two column tiles of
          // its first k-step in the last two units (16 each).
          if (s == 0) {
            if (q & 1) dequant_tile<SWIGLU, 4, 4>(raw, q >> 1, 1, ss, fn);
            else dequant_tile<SWIGLU, 0, 4>(raw, q >> 1, 1, ss, fn);
          } else if (q >= 4 - NU) {
#pragma unroll
            for (int t = 0; t < TPU; ++t)
              dequant_tile<SWIGLU>(raw, (q - (4 - NU)) * TPU + t, 0, ss_next, fn);
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (s == 0) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            else if (q >= 4 - NU) __builtin_amdgcn_sched_group_barrier(0x002, 4 * TPU, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (grp < GROUPS) {
          // spread the LOADS loads of step g+NS-1 over the units before B(g+1)
          const int upto = (LOADS * (grp + 1)) / GROUPS;
#pragma unroll
          for (int j = 0; j < LOADS; ++j)
            if (j >= (LOADS * grp) / GROUPS && j < upto) is.load(j, dst, wv);
          if (grp == GROUPS - 1) advance<BK, SWIGLU, W8>(is, a, tt, sc, nk, wv, lane);
        }
        if (s < KS - 1 && q < S1) {
          // fragments of the next k-step of this step, spread over S1 units
          if constexpr (!W8)
            if (q == 0) read_b<BK, SWIGLU>(cur, s + 1, wv, lane, fn);
          read_a<BK, W8>(cur, s + 1, wv, lane, fn, q * R1, R1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (W8) ss = ss_next;
  }
}

template <int BK, int NS, bool SWIGLU, bool W8>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_persist_kernel(GroupedGemmArgs args) {
  using G = Geo<BK, W8>;
  // one LDS object: the stages, then the tile table
  __shared__ __attribute__((aligned(1024))) char smem[NS * G::STAGE_BYTES + sizeof(TileTab)];
  char(*st)[G::STAGE_BYTES] = (char(*)[G::STAGE_BYTES])smem;
  TileTab& tt = *(TileTab*)(smem + NS * G::STAGE_BYTES);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int CN = SWIGLU ? BN / 2 : BN;

  // per-group M-tile prefix and row offsets, in LDS for the whole kernel
  const int total_m =
      group_tile_prefix<NTHR>(args.offsets, args.n_groups, BM, tt.ts, tt.off, tt.scan);
  __syncthreads();

  Sched sc;
  sc.n_groups = args.n_groups;
  sc.CN = CN;
  sc.ntn = (args.Nout + CN - 1) / CN;
  sc.nslot = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  sc.slot = blockIdx.x / kNumXcd;
  // A folded shared expert (the last group, B0x set) is spread over the
  // XCDs by M-tiles; otherwise every group's tiles are cut into one range
  // per XCD.
  const bool fold = args.B0x != nullptr;
  const int ms = fold ? tt.ts[sc.n_groups] - tt.ts[sc.n_groups - 1] : 0;
  const int routed = (total_m - ms) * sc.ntn;
  const int rper = (routed + kNumXcd - 1) / kNumXcd;
  sc.rlo = xcd * rper;
  sc.rcnt = max(0, min(rper, routed - sc.rlo));
  const int msper = (ms + kNumXcd - 1) / kNumXcd;
  sc.smlo = xcd * msper;
  sc.scnt = max(0, min(msper, ms - sc.smlo)) * sc.ntn;
  const int cnt = sc.rcnt + sc.scnt;
  if (sc.slot >= cnt) return;
  sc.ntile = (cnt - sc.slot + sc.nslot - 1) / sc.nslot;
  const int nk = args.K / BK;

  // tile 0's row indices, then the sources of its first steps
  Tile t = sched_tile(tt, sc, 0);
  if (args.row_index) {
    fetch_rows(args, tt, 0, t, wv, lane);
    wait_vm_lgkm<0>();
    __syncthreads();
  }
  Issuer<BK, SWIGLU, W8> is;
  is.it = 0;
  is.kt = 0;
  is.build(args, tt, t, wv, lane);
  if (args.row_index && sc.ntile > 1)
    fetch_rows(args, tt, 1, sched_tile(tt, sc, 1), wv, lane);
  // steps 0 .. NS-2 into stages 0 .. NS-2
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) is.load(j, st[s], wv);
    advance<BK, SWIGLU, W8>(is, args, tt, sc, nk, wv, lane);
  }
  // The row indices of the tile after the next are fetched when the issuer
  // enters a tile and read when it enters the next one.  The fetch has landed
  // for every wave after the first wait (at most (NS-2)*LOADS newer loads
  // outstanding) and barrier that follow NS-2 more steps of loads; the issuer
  // enters the next tile during the step nk later, before that step's barrier,
  // and the prologue enters tile 1 before B(0) unless nk >= NS.  So nk >= NS,
  // which the launchers check.
  wait_vm_lgkm<(NS - 2) * G::LOADS>();
  __builtin_amdgcn_s_barrier();  // B(0)

  constexpr int MB = Lay<W8>::MB, NT = Lay<W8>::NT;
  Frags<W8> f[2];
  u32x4_t raw[Lay<true>::NT];
  TileScale tsc{}, tsn{};
  StepScale ss{0.f, 0.f};
  if constexpr (W8) {
    tsc = tile_scale<SWIGLU>(args, t, wv);
    ss = step_scale(tsc, 0);
    read_w8_raw<BK, SWIGLU>(st[0], wv, lane, raw);
    read_a<BK, true>(st[0], 0, wv, lane, f[0]);
#pragma unroll
    for (int j = 0; j < NT; ++j) dequant_tile<SWIGLU>(raw, j, 0, ss, f[0]);
  } else {
    read_b<BK, SWIGLU>(st[0], 0, wv, lane, f[0]);
    read_a<BK, false>(st[0], 0, wv, lane, f[0]);
  }
  f32x16_t acc[MB][NT];
  int g = 0;
  for (int i = 0; i < sc.ntile; ++i) {
    if (i > 0) {
      t = sched_tile(tt, sc, i);
      if constexpr (W8) tsc = tsn;
    }
    if constexpr (W8)
      tsn = i + 1 < sc.ntile
                ? tile_scale<SWIGLU>(args, sched_tile(tt, sc, i + 1), wv)
                : tsc;
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[r][c][e] = 0.f;
    run_tile<BK, NS, SWIGLU, W8>(g, nk, is, args, tt, sc, st, wv, lane, f, acc, tsc, tsn,
                                 ss, raw);
    store_tile<SWIGLU, W8>(args, t, wv, lane, acc);
  }
  // no load may still be writing LDS when the workgroup ends
  wait_vm_lgkm<0>();
}

// stages: fp8 weights with 4, 5 and 6 stages measured 12.49, 12.47-12.59 and
// 12.52-12.69 ms on the routed up + down GEMMs of the V3-shaped prefill
constexpr int LIB_BK = 32, LIB_NS = 4, LIB_BK_W8 = 32, LIB_NS_W8 = 4;

}  // namespace gp

MOE_CHECKS_READER(gemm_persist)

int persist_grid() {
  // per device: the CU count of each GPU the library runs on, read once
  constexpr int kMaxDev = 64;
  static std::atomic<int> grid[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = -1;
  if (dev >= 0) {
    const int g = grid[dev].load(std::memory_order_relaxed);
    if (g > 0) return g;
  }
  int cus = 0;
  if (dev < 0 ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < kNumXcd)
    cus = 256;
  const int g = (cus / kNumXcd) * kNumXcd;
  if (dev >= 0) grid[dev].store(g, std::memory_order_relaxed);
  return g;
}

int persist_min_k(bool fp8_weights) {
  return fp8_weights ? gp::LIB_NS_W8 * gp::LIB_BK_W8 : gp::LIB_NS * gp::LIB_BK;
}

hipError_t launch_gemm_bf16_persist(const GroupedGemmArgs& a, bool swiglu, hipStream_t s) {
  if (a.max_rows <= 0 || a.n_groups <= 0) return hipSuccess;
  if (a.K % gp::LIB_BK != 0 || a.K < persist_min_k(false)) return hipErrorInvalidValue;
  const int grid = persist_grid();
  if (swiglu)
    gp::gemm_bf16_persist_kernel<gp::LIB_BK, gp::LIB_NS, true, false><<<grid, gp::NTHR, 0, s>>>(a);
  else
    gp::gemm_bf16_persist_kernel<gp::LIB_BK, gp::LIB_NS, false, false><<<grid, gp::NTHR, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_persist(const GroupedGemmArgs& a, bool swiglu, hipStream_t s) {
  if (a.max_rows <= 0 || a.n_groups <= 0) return hipSuccess;
  if (a.K % gp::LIB_BK_W8 != 0 || a.K < persist_min_k(true)) return hipErrorInvalidValue;
  const int grid = persist_grid();
  if (swiglu)
    gp::gemm_bf16_persist_kernel<gp::LIB_BK_W8, gp::LIB_NS_W8, true, true><<<grid, gp::NTHR, 0, s>>>(a);
  else
    gp::gemm_bf16_persist_kernel<gp::LIB_BK_W8, gp::LIB_NS_W8, false, true><<<grid, gp::NTHR, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
