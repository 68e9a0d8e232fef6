// Counting-sort permutation of (token, expert) slots on gfx950.
//
// The reference forward shown on open-model-atlas ("DeepSeek-V3.2-Exp -
// Mixture of experts", code excerpt of the MoE forward) counts the tokens of
// every expert with a bincount, skips experts with none, and gathers each
// expert's rows with a where/index pair.  Here the same grouping is one stable
// counting sort on the device (no host round trip):
//   1. hist:    one wavefront per chunk of 256 slots counts its experts in LDS
//               and records each slot's rank among equal experts of the chunk
//               (64 slots at a time: one ballot per bit of the expert id gives
//               each lane the lanes of its expert; popcounts give the rank);
//   2. scan:    one block per expert scans the chunk counts -> per-chunk base
//               and the expert's total;
//   3. scatter: row = offset[e] + base[chunk][e] + rank; row_token / slot_row.
// Up to four chunks (decode) run all three steps in one block.
// Rows are ordered by expert, then by slot index f = t*k + j (stable).
#include "moe_internal.h"
#include "wave_utils.h"

namespace moe {

// Expert ids outside [0, N) are clamped to 0 or N-1 wherever they address
// memory, the same way in every kernel: a bad id then routes its slot to the
// nearest valid expert instead of indexing past the counts, the offsets or
// the row maps.
__device__ __forceinline__ int clamp_expert(int e, int N) {
  MOE_DCHECK(e >= 0 && e < N, kCheckExpertId);
  return e < 0 ? 0 : (e >= N ? N - 1 : e);
}

// Wavefront-level: counts of chunk c's experts into cnt (LDS, N entries,
// zeroed) and each slot's rank among the equal experts of the chunk.
__device__ __forceinline__ void rank_chunk(const int32_t* __restrict__ idx, int64_t S, int N,
                                           int c, int* cnt, int32_t* rank) {
  const int lane = lane_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int it = 0; it < kPermChunk / 64; ++it) {
    const int64_t f = (int64_t)c * kPermChunk + it * 64 + lane;
    const bool valid = f < S;
    const int e = valid ? clamp_expert(idx[f], N) : 0;
    // the lanes holding the same expert, from one ballot per bit of the id
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kPermIdBits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t m = __ballot(valid && set);
      peers &= set ? m : ~m;
    }
    const int before = __popcll(peers & lt_mask);  // equal experts in earlier slots
    const int base = valid ? cnt[e] : 0;
    __builtin_amdgcn_wave_barrier();
    // the first lane of each expert advances its count
    if (valid && before == 0) cnt[e] = base + __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (valid) rank[f] = base + before;
  }
}

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ idx,
                                                           int64_t S, int N, int nchunks,
                                                           int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ rank) {
  extern __shared__ int cnt_all[];  // 4 * N
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int c = blockIdx.x * 4 + w;
  int* cnt = cnt_all + w * N;
  for (int i = lane; i < N; i += 64) cnt[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  if (c >= nchunks) return;
  rank_chunk(idx, S, N, c, cnt, rank);
  for (int i = lane; i < N; i += 64) hist[(int64_t)c * N + i] = cnt[i];
}

// A few slots (decode: S <= 4 chunks): one block does all three steps, wave w
// ranking chunk w, with the counts and ranks kept in LDS.
__global__ __launch_bounds__(256) void permute_small_kernel(
    const int32_t* __restrict__ idx, int64_t S, int k, int N, int nchunks,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row) {
  __shared__ int cnt[4][256];            // per chunk, then the chunk's base per expert
  __shared__ int rank_s[4 * kPermChunk];
  __shared__ int s_off[257];
  __shared__ int scratch[4];
  const int tid = threadIdx.x, w = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) cnt[i >> 8][i & 255] = 0;
  __syncthreads();
  if (w < nchunks) rank_chunk(idx, S, N, w, cnt[w], rank_s);
  __syncthreads();
  int v = 0;
  if (tid < N) {
    for (int c = 0; c < nchunks; ++c) {
      const int x = cnt[c][tid];
      cnt[c][tid] = v;
      v += x;
    }
  }
  int tot;
  const int incl = block_incl_scan<256>(v, scratch, &tot);
  if (tid < N) {
    s_off[tid] = incl - v;
    counts[tid] = v;
    offsets[tid] = incl - v;
  }
  if (tid == 0) {
    s_off[N] = tot;
    offsets[N] = tot;
    MOE_DCHECK(tot == S, kCheckOffsets);
  }
  __syncthreads();
  for (int64_t f = tid; f < S; f += 256) {
    const int e = clamp_expert(idx[f], N);
    const int row = s_off[e] + cnt[f / kPermChunk][e] + rank_s[f];
    row_token[row] = (int32_t)(f / k);
    slot_row[f] = row;
  }
}

__global__ __launch_bounds__(256) void permute_scan_kernel(const int32_t* __restrict__ hist,
                                                           int nchunks, int N,
                                                           int32_t* __restrict__ base,
                                                           int32_t* __restrict__ counts) {
  __shared__ int scratch[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < nchunks ? hist[(int64_t)c * N + e] : 0;
    int tot;
    const int incl = block_incl_scan<256>(v, scratch, &tot);
    if (c < nchunks) base[(int64_t)c * N + e] = carry + incl - v;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// One block per chunk of 256 slots; every block rebuilds the expert offsets
// from counts (N <= 256) and block 0 publishes them.
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t S, int k, int N, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row) {
  __shared__ int s_off[257];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const int v = tid < N ? counts[tid] : 0;
  int tot;
  const int incl = block_incl_scan<256>(v, scratch, &tot);
  if (tid < N) s_off[tid] = incl - v;
  if (tid == 0) s_off[N] = tot;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < N) offsets[tid] = s_off[tid];
    if (tid == 0) offsets[N] = tot;
    if (tid == 0) MOE_DCHECK(tot == S, kCheckOffsets);
  }
  const int64_t f = (int64_t)blockIdx.x * kPermChunk + tid;
  if (f >= S) return;
  const int e = clamp_expert(idx[f], N);
  const int row = s_off[e] + base[(int64_t)blockIdx.x * N + e] + rank[f];
  row_token[row] = (int32_t)(f / k);
  slot_row[f] = row;
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int N, int32_t* hist,
                          int32_t* base, int32_t* rank, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, hipStream_t stream) {
  const int64_t S = T * k;
  const int nchunks = (int)cdiv(S, kPermChunk);
  if (nchunks <= 4) {
    permute_small_kernel<<<1, 256, 0, stream>>>(idx, S, k, N, nchunks, counts, offsets, row_token,
                                                slot_row);
    return hipGetLastError();
  }
  permute_hist_kernel<<<(unsigned)cdiv(nchunks, 4), 256, 4 * N * sizeof(int), stream>>>(
      idx, S, N, nchunks, hist, rank);
  permute_scan_kernel<<<N, 256, 0, stream>>>(hist, nchunks, N, base, counts);
  permute_scatter_kernel<<<nchunks, 256, 0, stream>>>(idx, S, k, N, counts, base, rank, offsets,
                                                      row_token, slot_row);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void set_range_kernel(int32_t* p, int32_t n) {
  if (threadIdx.x == 0) {
    p[0] = 0;
    p[1] = n;
  }
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(unsigned)cdiv(n, 256), 256, 0, stream>>>(p, n, value);
  return hipGetLastError();
}

hipError_t launch_set_range(int32_t* p, int32_t n, hipStream_t stream) {
  set_range_kernel<<<1, 64, 0, stream>>>(p, n);
  return hipGetLastError();
}

// The shared expert as one more group after the routed slots: its rows are
// every token in order, and the group ends at slots + T.
__global__ void append_shared_rows_kernel(int32_t* __restrict__ row_token_tail, int32_t T,
                                          int32_t* __restrict__ offsets_last, int32_t end) {
  const int32_t t = (int32_t)blockIdx.x * 256 + threadIdx.x;
  if (t < T) row_token_tail[t] = t;
  if (t == 0) offsets_last[0] = end;
}

hipError_t launch_append_shared_rows(int32_t* row_token_tail, int32_t T, int32_t* offsets_last,
                                     int32_t end, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  append_shared_rows_kernel<<<(unsigned)cdiv(T, 256), 256, 0, stream>>>(row_token_tail, T,
                                                                        offsets_last, end);
  return hipGetLastError();
}

// x_perm[r] = x[row_token[r]]: one 256-thread block per row, 16-byte copies.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          u32x4_t* __restrict__ out,
                                                          int64_t vec_per_row) {
  const int64_t r = blockIdx.x;
  const int64_t src = row_token[r];
  for (int64_t i = threadIdx.x; i < vec_per_row; i += 256)
    out[r * vec_per_row + i] = x[src * vec_per_row + i];
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, void* x_perm,
                              int64_t rows, int64_t row_bytes, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  gather_rows_kernel<<<(unsigned)rows, 256, 0, stream>>>((const u32x4_t*)x, row_token,
                                                         (u32x4_t*)x_perm, row_bytes / 16);
  return hipGetLastError();
}

MOE_CHECKS_READER(permute)

}  // namespace moe
