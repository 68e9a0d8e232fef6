// Router of the DeepSeekMoE layer on gfx950.
//
// Logits z = x W_r (open-model-atlas, DeepSeek-V3.2-Exp "Mixture of experts",
// "All 19 steps", router; aiany.app explainer Step 2: the dot product of the
// token with every expert's centroid), then per token: softmax over the routed
// experts or sigmoid scores, group-limited top-k with lower-index tie-breaks,
// and the gates (G = scale * p_sel, or G = scale * s_sel / sum s_sel).
#include "moe_internal.h"
#include "wave_utils.h"

namespace moe {

// ---------------------------------------------------------------------------
// z[T, N] = x[T, d] . W_r[N, d]^T, fp32 FMA in k order.  64 x 64 tile per
// 256-thread block, 4 x 4 outputs per thread, d % 32 == 0.
// ---------------------------------------------------------------------------
template <typename TX>
__global__ __launch_bounds__(256) void router_logits_simt_kernel(const TX* __restrict__ x,
                                                                 const float* __restrict__ W,
                                                                 float* __restrict__ z, int64_t T,
                                                                 int d, int N) {
  __shared__ float xs[32][64 + 4];
  __shared__ float ws[32][64 + 4];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
  const int tm = tid >> 4, tn = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += 32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 5, kk = e & 31;
      const int64_t row = m0 + r;
      xs[kk][r] = row < T ? ElemIO<TX>::load(x + row * d + k0 + kk) : 0.f;
      const int n = n0 + r;
      ws[kk][r] = n < N ? W[(int64_t)n * d + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + tm * 4 + i;
    if (row >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn * 4 + j;
      if (n < N) z[row * N + n] = acc[i][j];
    }
  }
}

hipError_t launch_router_logits_simt(bool x_bf16, const void* x, const float* W_r, float* z,
                                     int64_t T, int d, int N, hipStream_t stream) {
  dim3 grid((unsigned)cdiv(T, 64), (unsigned)cdiv(N, 64));
  if (x_bf16)
    router_logits_simt_kernel<bf16_t><<<grid, 256, 0, stream>>>((const bf16_t*)x, W_r, z, T, d, N);
  else
    router_logits_simt_kernel<float><<<grid, 256, 0, stream>>>((const float*)x, W_r, z, T, d, N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// z = x W_r on MFMA (x bf16).  W_r is fp32; every weight is split exactly into
// three bf16 parts hi + mid + lo (successive round-to-nearest residuals: 8+8+8
// significand bits cover fp32's 24), and each bf16 x bf16 product is exact in
// the fp32 accumulator, so three v_mfma_f32_32x32x16_bf16 per fragment pair
// give the fp32 dot product.  The split is done once per call into three bf16
// planes of W_r's shape (router_split_kernel), not by every block that reads
// a W_r tile.  128 tokens x 128 experts per 256-thread block, K staged 64 at
// a time; blockIdx.z splits K (partial sums in zpart[z], added in split order
// by the selection kernel) so that small token counts still fill the GPU.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {  // finite inputs
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
}

// The three bf16 parts (hi, mid, lo) of four fp32 weights, four packed bf16
// per part.
__device__ __forceinline__ void split3(const f32x4_t& w, u32x2_t (&part)[3]) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = bf16_rne_bits(w[e]);
    const float r1 = w[e] - __uint_as_float(h[e]);
    m[e] = bf16_rne_bits(r1);
    l[e] = bf16_rne_bits(r1 - __uint_as_float(m[e]));
  }
  part[0] = u32x2_t{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3]};
  part[1] = u32x2_t{(m[0] >> 16) | m[1], (m[2] >> 16) | m[3]};
  part[2] = u32x2_t{(l[0] >> 16) | l[1], (l[2] >> 16) | l[3]};
}

// planes[p * n + i] = part p of W[i] (n = N * d, a multiple of 4)
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ W,
                                                           bf16_t* __restrict__ planes, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  u32x2_t part[3];
  split3(*(const f32x4_t*)(W + i), part);
#pragma unroll
  for (int p = 0; p < 3; ++p) *(u32x2_t*)(planes + p * n + i) = part[p];
}

// PRESPLIT: W points at the three bf16 planes; else at W_r (fp32), which each
// block splits while it stages its tiles.  Many token blocks (prefill) share
// every W_r tile, so the planes are made once; with one or two (decode) the
// in-block split costs less than a pass over W_r.  With the planes, K is
// staged 32 at a time (64 KiB of LDS, two blocks per CU, so one block's
// loads and barrier overlap the other's MFMAs); the in-block split stages 64.
template <bool PRESPLIT>
__global__ __launch_bounds__(256, PRESPLIT ? 2 : 1) void router_logits_mfma_kernel(
    const bf16_t* __restrict__ x, const void* __restrict__ W, float* __restrict__ zpart,
    int64_t T, int d, int N, int nsplit) {
  constexpr int BM = 128, BN = 128, BK = PRESPLIT ? 32 : 64;
  constexpr int CPR = BK / 8;           // 16-byte chunks per LDS row
  constexpr int AC = BM * CPR / 256;    // activation chunks per thread
  // chunk c of row r sits at chunk swz(r, c): the 16 rows a quarter-wave reads
  // with one ds_read_b128 fall on distinct banks (64-byte rows: 4 rows per
  // 256 bytes, so rows 4 apart are told apart; 128-byte rows: 2 per 256)
  auto swz = [](int r, int c) { return PRESPLIT ? c ^ ((r >> 2) & 3) : c ^ (r & 7); };
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b[2][3][BN * BK];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int nk = d / BK;
  const int kt0 = (int)((int64_t)blockIdx.z * nk / nsplit);
  const int kt1 = (int)((int64_t)(blockIdx.z + 1) * nk / nsplit);

  // activation tile: 128 rows x BK bf16 = CPR chunks of 16 B per row, AC per
  // thread, swizzled by row in LDS
  const bf16_t* a_src[AC];
  int a_lds[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + 256 * i;
    const int r = c / CPR, col = c % CPR;
    int64_t gr = m0 + r;
    if (gr > T - 1) gr = T - 1;
    a_src[i] = x + gr * d + col * 8;
    a_lds[i] = r * BK + (swz(r, col) << 3);
  }
  // W_r tile, 128 expert rows x BK.  Planes: the activation tile's geometry,
  // AC chunks per thread and plane.  fp32 (BK = 64): 16 chunks of 4 floats per
  // row, 8 per thread, split into the planes on the way into LDS.
  constexpr int NB = PRESPLIT ? AC : 8;
  const char* b_src[NB];
  int b_lds[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int c = tid + 256 * i;
    const int r = PRESPLIT ? c / CPR : c >> 4;
    int n = n0 + r;
    if (n > N - 1) n = N - 1;
    if constexpr (PRESPLIT) {
      const int col = c % CPR;
      b_src[i] = (const char*)((const bf16_t*)W + (int64_t)n * d + col * 8);
      b_lds[i] = r * BK + (swz(r, col) << 3);
    } else {
      const int q = c & 15;  // 4-float group within the 64-wide K tile
      b_src[i] = (const char*)((const float*)W + (int64_t)n * d + q * 4);
      b_lds[i] = r * BK + (swz(r, q >> 1) << 3) + (q & 1) * 4;
    }
  }
  const int64_t pbytes = (int64_t)N * d * 2;  // bytes per plane
  u32x4_t ra[AC], rb[PRESPLIT ? 3 : 1][NB];
  auto gload = [&](int kt) {
    const int ko = kt * BK;
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = *(const u32x4_t*)(a_src[i] + ko);
#pragma unroll
    for (int p = 0; p < (PRESPLIT ? 3 : 1); ++p)
#pragma unroll
      for (int i = 0; i < NB; ++i)
        rb[p][i] = *(const u32x4_t*)(b_src[i] + p * pbytes + (int64_t)ko * (PRESPLIT ? 2 : 4));
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AC; ++i) *(u32x4_t*)(&lds_a[buf][a_lds[i]]) = ra[i];
    if constexpr (PRESPLIT) {
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < NB; ++i) *(u32x4_t*)(&lds_b[buf][p][b_lds[i]]) = rb[p][i];
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        u32x2_t part[3];
        split3(__builtin_bit_cast(f32x4_t, rb[0][i]), part);
#pragma unroll
        for (int p = 0; p < 3; ++p) *(u32x2_t*)(&lds_b[buf][p][b_lds[i]]) = part[p];
      }
    }
  };

  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int l32 = lane & 31, khalf = lane >> 5;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(kt0);
  lstore(0);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    if (kt + 1 < kt1) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = 2 * ks + khalf;
      bf16x8_t af[2], bfr[3][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + l32;
        af[i] = *(const bf16x8_t*)(&lds_a[cur][r * BK + (swz(r, chunk) << 3)]);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wn * 64 + j * 32 + l32;
          bfr[p][j] = *(const bf16x8_t*)(&lds_b[cur][p][r * BK + (swz(r, chunk) << 3)]);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int p = 0; p < 3; ++p)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[p][j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < kt1) lstore(cur ^ 1);
    __syncthreads();
  }
  float* __restrict__ zp = zpart + (int64_t)blockIdx.z * T * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (row >= T) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + l32;
        if (col < N) zp[row * N + col] = acc[i][j][r];
      }
    }
}

// About 512 blocks in all, each with at least two K tiles, and at most
// kRouterSelectSplits partials (added in split order by the selection kernel,
// at most 64 MiB of them).  A few tokens (decode) thus spread over many
// blocks: a block's K loop waits for one load per tile, so fewer tiles per
// block is what makes it fast.
int router_mfma_splits(int64_t T, int d, int N) {
  const int64_t tiles = cdiv(T, 128) * cdiv(N, 128);
  if (tiles <= 0) return 1;
  const int nk = d / 64;
  int64_t s = cdiv(512, tiles);
  if (s > nk / 2) s = nk / 2;
  if (s > kRouterSelectSplits) s = kRouterSelectSplits;
  const int64_t per_split = T * (int64_t)N * 4;
  if (s * per_split > (int64_t(64) << 20)) s = (int64_t(64) << 20) / per_split;
  if (s < 1) s = 1;
  return (int)s;
}

bool router_presplit(int64_t T) { return cdiv(T, 128) >= kRouterPresplitBlocks; }

hipError_t launch_router_logits_mfma(const bf16_t* x, const float* W_r, bf16_t* planes,
                                     float* zpart, int64_t T, int d, int N, int nsplit,
                                     hipStream_t stream) {
  dim3 grid((unsigned)cdiv(T, 128), (unsigned)cdiv(N, 128), (unsigned)nsplit);
  if (router_presplit(T)) {
    router_split_kernel<<<(unsigned)cdiv((int64_t)N * d / 4, 256), 256, 0, stream>>>(
        W_r, planes, (int64_t)N * d);
    router_logits_mfma_kernel<true><<<grid, 256, 0, stream>>>(x, planes, zpart, T, d, N, nsplit);
  } else {
    router_logits_mfma_kernel<false><<<grid, 256, 0, stream>>>(x, W_r, zpart, T, d, N, nsplit);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection: one wavefront per token.  Lane l holds experts l, l+64, l+128,
// l+192 (N <= 256).  Keys are compared as (ordered key << 32 | ~index), so a
// 64-bit max picks the larger key and, on equal keys, the lower index.
// ---------------------------------------------------------------------------
constexpr int kSelPerLane = 4;

__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  return ((uint64_t)f32_to_ordered(key) << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ int unpack_idx(uint64_t p) {
  return (int)(0xffffffffu - (uint32_t)(p & 0xffffffffu));
}

// Group scores when a group is 2^STEPS consecutive experts (2..64): group
// j * (64 >> STEPS) + lane >> STEPS is a segment of lanes of register j, so
// all groups find their top entries at once with segmented maxima.  Each
// group's score adds its group_topn largest keys, largest first, from 0.
// Returns, in lane g < n_groups, the score of group g.
template <int STEPS>
__device__ __forceinline__ float group_scores_segmented(const float (&key)[kSelPerLane],
                                                        const bool (&ok)[kSelPerLane], int lane,
                                                        int n_groups, int group_topn) {
  constexpr int GS = 1 << STEPS, SEG = 64 / GS;  // lanes per group, groups per register
  float s[kSelPerLane];
  unsigned taken = 0;
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) s[j] = 0.f;
  for (int r = 0; r < group_topn; ++r) {
    uint64_t best[kSelPerLane];
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      best[j] = ok[j] && !((taken >> j) & 1u) ? pack_key(key[j], lane + 64 * j) : 0;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) best[j] = segment_max_u64<STEPS>(best[j]);
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      if (best[j] != 0 && (unpack_idx(best[j]) & 63) == lane) taken |= 1u << j;
      s[j] += ordered_to_f32((uint32_t)(best[j] >> 32));
    }
  }
  float mine = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) {
    const float v = __shfl(s[j], (lane % SEG) * GS, 64);
    if (lane < n_groups && lane / SEG == j) mine = v;
  }
  return mine;
}

// R > 0 (N % 4 == 0): lane l adds the partials of experts 4l .. 4l+3 with
// 16-byte loads, R splits in flight at a time, and the sums go through LDS to
// the lanes that select.  R == 0: one expert per load, 8 splits at a time.
// Either way each expert's partials are added in split order, starting from 0.
template <int R>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ z, int nsplit, const float* __restrict__ b, int64_t T, int N, int k,
    int n_groups, int topk_groups, int group_topn, int gate, float route_scale, ExpertMask mask,
    int32_t* __restrict__ out_idx, float* __restrict__ out_gate, float* __restrict__ scores) {
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
  if (t >= T) return;  // uniform per wavefront
  const float NEG_INF = -__builtin_inff();

  float val[kSelPerLane], key[kSelPerLane];
  bool ok[kSelPerLane];
  // the bias first (a missing bias reads z and is not used), so that its
  // loads overlap those of the partials
  float bias[kSelPerLane];
  const float* bsrc = b ? b : z;
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) {
    ok[j] = lane + 64 * j < N;
    bias[j] = bsrc[ok[j] ? lane + 64 * j : 0];
  }
  float zsum[kSelPerLane];
  if (R > 0) {
    __shared__ __attribute__((aligned(16))) float sums[4][256];
    // lanes past the last expert read experts 0..3 and drop them
    const float* zp = z + t * N + (4 * lane < N ? 4 * lane : 0);
    const int64_t sstride = T * (int64_t)N;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += (R > 0 ? R : 1)) {
      f32x4_t part[R > 0 ? R : 1];
#pragma unroll
      for (int sp = 0; sp < R; ++sp) {  // clamped, so that no load is conditional
        const int sx = s0 + sp < nsplit ? s0 + sp : nsplit - 1;
        part[sp] = *(const f32x4_t*)(zp + sx * sstride);
      }
      __builtin_amdgcn_sched_barrier(0);  // all R loads before the first add
#pragma unroll
      for (int sp = 0; sp < R; ++sp) {
        const f32x4_t a = acc + part[sp];
        acc = s0 + sp < nsplit ? a : acc;
      }
    }
    *(f32x4_t*)&sums[wv][4 * lane] = acc;  // this wavefront's row only
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) zsum[j] = sums[wv][lane + 64 * j];
  } else {
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) zsum[j] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      float part[kSelPerLane][8];
#pragma unroll
      for (int j = 0; j < kSelPerLane; ++j)
#pragma unroll
        for (int sp = 0; sp < 8; ++sp)
          part[j][sp] = ok[j] && s0 + sp < nsplit
                            ? z[((int64_t)(s0 + sp) * T + t) * N + lane + 64 * j]
                            : 0.f;
#pragma unroll
      for (int j = 0; j < kSelPerLane; ++j)
#pragma unroll
        for (int sp = 0; sp < 8; ++sp)
          if (s0 + sp < nsplit) zsum[j] += part[j][sp];
    }
  }
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) {
    const int e = lane + 64 * j;
    const float zz = zsum[j];
    const float bb = (ok[j] && b) ? bias[j] : 0.f;
    val[j] = zz + bb;  // softmax: biased logit; overwritten below for sigmoid
    key[j] = bb;
    if (gate == 1) {
      const float s = 1.f / (1.f + expf(-zz));
      val[j] = s;
      key[j] = s + bb;
    }
  }
  if (gate == 0) {
    float m = NEG_INF;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (ok[j]) m = fmaxf(m, val[j]);
    m = wave_max(m);
    float ex[kSelPerLane], sum = 0.f;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      ex[j] = ok[j] ? expf(val[j] - m) : 0.f;
      sum += ex[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      val[j] = ex[j] / sum;
      key[j] = val[j];
    }
  }
  if (scores) {
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (ok[j]) scores[t * N + lane + 64 * j] = val[j];
  }
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j)
    if (!ok[j]) key[j] = NEG_INF;

  // ---- experts taken out of the selection (aiany.app explainer, Step 9,
  // probe 1): a fixed set, then each token's mask_top highest remaining keys
  // (same order as the top-k: key descending, index ascending).  The scores
  // written above are unchanged.
  if (mask.any) {
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (!((mask.allow[j] >> lane) & 1ull)) key[j] = NEG_INF;
  }
  for (int r = 0; r < mask.top; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (key[j] != NEG_INF) {
        const uint64_t p = pack_key(key[j], lane + 64 * j);
        best = p > best ? p : best;
      }
    best = wave_max_u64(best);
    const int e_sel = unpack_idx(best);
    if ((e_sel & 63) == lane) {
#pragma unroll
      for (int j = 0; j < kSelPerLane; ++j)
        if (j == (e_sel >> 6)) key[j] = NEG_INF;
    }
  }

  // ---- group limit: score = sum of the group_topn largest keys of the group
  if (n_groups > 1) {
    const int gs = N / n_groups;
    int grp[kSelPerLane];
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) grp[j] = (lane + 64 * j) / gs;
    float my_gscore = NEG_INF;
    switch (gs) {
      case 2: my_gscore = group_scores_segmented<1>(key, ok, lane, n_groups, group_topn); break;
      case 4: my_gscore = group_scores_segmented<2>(key, ok, lane, n_groups, group_topn); break;
      case 8: my_gscore = group_scores_segmented<3>(key, ok, lane, n_groups, group_topn); break;
      case 16: my_gscore = group_scores_segmented<4>(key, ok, lane, n_groups, group_topn); break;
      case 32: my_gscore = group_scores_segmented<5>(key, ok, lane, n_groups, group_topn); break;
      case 64: my_gscore = group_scores_segmented<6>(key, ok, lane, n_groups, group_topn); break;
      default:  // one group at a time over the whole wavefront
        for (int g = 0; g < n_groups; ++g) {
          unsigned taken = 0;
          float s = 0.f;
          for (int r = 0; r < group_topn; ++r) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < kSelPerLane; ++j) {
              if (ok[j] && grp[j] == g && !((taken >> j) & 1u)) {
                const uint64_t p = pack_key(key[j], lane + 64 * j);
                best = p > best ? p : best;
              }
            }
            best = wave_max_u64(best);
            const int e_sel = unpack_idx(best);
            if ((e_sel & 63) == lane) taken |= 1u << (e_sel >> 6);
            s += ordered_to_f32((uint32_t)(best >> 32));
          }
          if (lane == g) my_gscore = s;
        }
    }
    uint64_t allowed = 0;
    for (int r = 0; r < topk_groups; ++r) {
      uint64_t p = 0;
      if (lane < n_groups && !((allowed >> lane) & 1ull)) p = pack_key(my_gscore, lane);
      p = wave_max_u64(p);
      allowed |= 1ull << unpack_idx(p);
    }
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (ok[j] && !((allowed >> grp[j]) & 1ull)) key[j] = NEG_INF;
  }

  // ---- top-k (k <= 64): lane i keeps the i-th selection
  unsigned taken = 0;
  int my_idx = 0;
  float my_val = 0.f;
  for (int i = 0; i < k; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      if (!((taken >> j) & 1u) && key[j] != NEG_INF) {
        const uint64_t p = pack_key(key[j], lane + 64 * j);
        best = p > best ? p : best;
      }
    }
    best = wave_max_u64(best);
    const int e_sel = unpack_idx(best);
    if (lane == (e_sel & 63)) taken |= 1u << (e_sel >> 6);
    if (lane == i) my_idx = e_sel;
  }
  // lane i < k fetches the value of its selection from the lane that holds it
  {
    float got[kSelPerLane];
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) got[j] = __shfl(val[j], my_idx & 63, 64);
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (j == (my_idx >> 6)) my_val = got[j];
  }
  float g_out = route_scale * my_val;
  if (gate == 1) {
    const float tot = wave_sum(lane < k ? my_val : 0.f);
    g_out = route_scale * my_val / tot;
  }
  if (lane < k) {
    MOE_DCHECK(my_idx >= 0 && my_idx < N && __builtin_isfinite(g_out), kCheckSelect);
    out_idx[t * k + lane] = my_idx;
    out_gate[t * k + lane] = g_out;
  }
}

hipError_t launch_router_select(const float* z, int nsplit, const float* b, int64_t T, int N, int k,
                                int n_groups, int topk_groups, int group_topn, int gate,
                                float route_scale, int32_t* idx, float* gates, float* scores,
                                hipStream_t stream, const ExpertMask* mask) {
  // one wavefront per token; a few tokens (decode) get a block each, so that
  // their loads of the partials spread over as many CUs
  const int wpb = T < 1024 ? 1 : 4;
  const unsigned blocks = (unsigned)cdiv(T, wpb);
  const ExpertMask m = mask ? *mask : ExpertMask{};
  const bool vec = N % 4 == 0 && ((uintptr_t)z & 15) == 0;
#define MOE_SELECT(R)                                                                          \
  router_select_kernel<R><<<blocks, 64 * wpb, 0, stream>>>(z, nsplit, b, T, N, k, n_groups,    \
                                                      topk_groups, group_topn, gate,           \
                                                      route_scale, m, idx, gates, scores)
  if (!vec) MOE_SELECT(0);
  else if (nsplit <= 2) MOE_SELECT(2);
  else if (nsplit <= 8) MOE_SELECT(8);
  else MOE_SELECT(32);
#undef MOE_SELECT
  return hipGetLastError();
}

// Auxiliary-loss-free balancing step (grasp.study lesson, 3.2): expert i's
// bias moves by gamma towards balance, up when its load is below the mean
// slots/N and down when above; the comparison N*load_i vs slots is exact.
__global__ void bias_update_kernel(float* __restrict__ b, const int32_t* __restrict__ counts,
                                   int N, int64_t slots, float gamma) {
  const int i = (int)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int64_t load = (int64_t)counts[i] * N;
  if (load < slots) b[i] = b[i] + gamma;
  else if (load > slots) b[i] = b[i] - gamma;
}

hipError_t launch_bias_update(float* b, const int32_t* counts, int N, int64_t slots, float gamma,
                              hipStream_t stream) {
  bias_update_kernel<<<(unsigned)cdiv(N, 256), 256, 0, stream>>>(b, counts, N, slots, gamma);
  return hipGetLastError();
}

MOE_CHECKS_READER(router)

}  // namespace moe
