// Device-side tile scheduling for the grouped (per-expert) GEMMs.
//
// The launch is sized on the host from an upper bound of the row count
// (max_rows / BM + n_groups M-tiles) and never waits for the real expert
// counts: every workgroup rebuilds the per-expert tile prefix from the device
// offsets in LDS, exits if its slot is past the real work, and otherwise maps
// its slot to (expert, N-tile, M-tile).  Experts with no rows own no tile, so
// their weights are never read.
//
// XCD-aware order: consecutive workgroup ids go round-robin over the 8 XCDs
// (each with its own L2), so slot w runs tile xcd(w) * per + w / 8.  Each XCD
// thereby walks one contiguous range of tiles, ordered expert-major, then
// N-tile, then M-tile: the M-tiles that share a weight N-tile are resident on
// the same XCD at the same time and read it through the same L2.
#pragma once
#include "moe_internal.h"
#include "wave_utils.h"

namespace moe {

constexpr int kMaxGroups = 512;  // routed experts (<= 256) + a folded shared expert
constexpr int kNumXcd = 8;

struct TileCoord {
  int group;
  int64_t row0;  // first row of the tile
  int64_t rend;  // end of the group's rows
  int n0;        // first output column
};

// ts[g] = number of BM-row tiles of groups 0..g-1 (ts[0] = 0), for up to
// kMaxGroups groups: thread t takes groups t*PER .. t*PER+PER-1.  If `off` is
// non-null it receives the group row offsets.  Returns the total; must be
// called by all NT threads of the block; ts/off are complete after a barrier.
template <int NT>
__device__ __forceinline__ int group_tile_prefix(const int32_t* __restrict__ offsets,
                                                 int n_groups, int BM, int* ts, int* off,
                                                 int* s_scratch /* NT/64 */) {
  constexpr int PER = (kMaxGroups + NT - 1) / NT;
  const int tid = threadIdx.x;
  int mt[PER];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    mt[q] = 0;
    if (g < n_groups) {
      const int o0 = offsets[g], o1 = offsets[g + 1];
      MOE_DCHECK(o0 >= 0 && o1 >= o0, kCheckGroupRows);
      mt[q] = (o1 - o0 + BM - 1) / BM;
      if (off) {
        off[g] = o0;
        if (g == n_groups - 1) off[g + 1] = o1;
      }
    }
    sum += mt[q];
  }
  int total;
  int run = block_incl_scan<NT>(sum, s_scratch, &total) - sum;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    run += mt[q];
    if (g < n_groups) ts[g + 1] = run;
  }
  if (tid == 0) ts[0] = 0;
  return total;
}

// Must be called by all NT threads of the block.  Returns false when the
// block has no tile (uniformly for the whole block).
template <int NT>
__device__ __forceinline__ bool grouped_tile_lookup(const int32_t* __restrict__ offsets,
                                                    int n_groups, int BM, int BN, int Nout,
                                                    int* s_ts /* kMaxGroups+1 */,
                                                    int* s_scratch /* NT/64 */, int* s_info,
                                                    TileCoord* tc) {
  const int tid = threadIdx.x;
  const int total_m = group_tile_prefix<NT>(offsets, n_groups, BM, s_ts, nullptr, s_scratch);
  const int n_tiles_n = (Nout + BN - 1) / BN;
  const int total = total_m * n_tiles_n;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int w = blockIdx.x;
  const int j = w / kNumXcd, xcd = w % kNumXcd;
  if (j >= per) return false;
  const int L = xcd * per + j;
  if (L >= total) return false;
  __syncthreads();
  for (int g = tid; g < n_groups; g += NT) {
    const int lo = s_ts[g] * n_tiles_n, hi = s_ts[g + 1] * n_tiles_n;
    if (L >= lo && L < hi) s_info[0] = g;
  }
  __syncthreads();
  const int g = s_info[0];
  const int tiles_g = s_ts[g + 1] - s_ts[g];
  const int rem = L - s_ts[g] * n_tiles_n;
  const int nt = rem / tiles_g, mt = rem % tiles_g;
  tc->group = g;
  tc->row0 = (int64_t)offsets[g] + (int64_t)mt * BM;
  tc->rend = offsets[g + 1];
  tc->n0 = nt * BN;
  return true;
}

// Upper bound of the number of workgroups a grouped launch needs.
inline int64_t grouped_grid(int64_t max_rows, int n_groups, int BM, int BN, int Nout) {
  const int64_t mt = max_rows / BM + n_groups;
  const int64_t n = mt * ((Nout + BN - 1) / BN);
  return ((n + kNumXcd - 1) / kNumXcd) * kNumXcd;
}

}  // namespace moe
