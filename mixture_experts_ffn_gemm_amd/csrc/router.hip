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

__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ z, const float* __restrict__ b, int64_t T, int N, int k,
    int n_groups, int topk_groups, int group_topn, int gate, float route_scale,
    int32_t* __restrict__ out_idx, float* __restrict__ out_gate, float* __restrict__ scores) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  const float NEG_INF = -__builtin_inff();

  float val[kSelPerLane], key[kSelPerLane];
  bool ok[kSelPerLane];
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) {
    const int e = lane + 64 * j;
    ok[j] = e < N;
    const float zz = ok[j] ? z[t * N + e] : 0.f;
    const float bb = (ok[j] && b) ? b[e] : 0.f;
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

  // ---- group limit: score = sum of the group_topn largest keys of the group
  if (n_groups > 1) {
    const int gs = N / n_groups;
    float my_gscore = NEG_INF;
    for (int g = 0; g < n_groups; ++g) {
      unsigned taken = 0;
      float s = 0.f;
      for (int r = 0; r < group_topn; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < kSelPerLane; ++j) {
          const int e = lane + 64 * j;
          if (ok[j] && e / gs == g && !((taken >> j) & 1u)) {
            const uint64_t p = pack_key(key[j], e);
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
    uint64_t allowed = 0;
    for (int r = 0; r < topk_groups; ++r) {
      uint64_t p = 0;
      if (lane < n_groups && !((allowed >> lane) & 1ull)) p = pack_key(my_gscore, lane);
      p = wave_max_u64(p);
      allowed |= 1ull << unpack_idx(p);
    }
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      const int e = lane + 64 * j;
      if (ok[j] && !((allowed >> (e / gs)) & 1ull)) key[j] = NEG_INF;
    }
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
    const int owner = e_sel & 63, jsel = e_sel >> 6;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (j == jsel) v = val[j];
    v = __shfl(v, owner, 64);
    if (lane == owner) taken |= 1u << jsel;
    if (lane == i) {
      my_idx = e_sel;
      my_val = v;
    }
  }
  float g_out = route_scale * my_val;
  if (gate == 1) {
    const float tot = wave_sum(lane < k ? my_val : 0.f);
    g_out = route_scale * my_val / tot;
  }
  if (lane < k) {
    out_idx[t * k + lane] = my_idx;
    out_gate[t * k + lane] = g_out;
  }
}

hipError_t launch_router_select(const float* z, const float* b, int64_t T, int N, int k,
                                int n_groups, int topk_groups, int group_topn, int gate,
                                float route_scale, int32_t* idx, float* gates, float* scores,
                                hipStream_t stream) {
  const unsigned blocks = (unsigned)cdiv(T, 4);
  router_select_kernel<<<blocks, 256, 0, stream>>>(z, b, T, N, k, n_groups, topk_groups,
                                                   group_topn, gate, route_scale, idx, gates,
                                                   scores);
  return hipGetLastError();
}

}  // namespace moe
