// Internal declarations shared by the gfx950 kernels and the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- device checks
// Compiled with MOE_DEVICE_CHECKS=1 (the checked library), kernels test the
// index invariants their memory accesses rely on and record a failure as a
// bit of their source file's flag word (an atomic OR through the vector memory
// path; nothing traps); where the index addresses memory a safe one replaces
// it.  Each source file's reader returns and clears its word after the device
// has finished.  Otherwise the checks compile to nothing.
#ifndef MOE_DEVICE_CHECKS
#define MOE_DEVICE_CHECKS 0
#endif
enum : unsigned {
  kCheckExpertId = 1u << 0,   // a top-k expert id outside [0, N) (permute clamps it)
  kCheckOffsets = 1u << 1,    // per-expert counts not adding up to the T*k slots
  kCheckRowIndex = 1u << 2,   // an activation row (gathered or not) outside the activation rows
  kCheckGroupRows = 1u << 3,  // group offsets negative or decreasing
  kCheckSlot = 1u << 4,       // a combine slot outside the T*k permuted rows
  kCheckSelect = 1u << 5,     // a selected expert outside [0, N) or a non-finite gate
};
#if MOE_DEVICE_CHECKS
static __device__ unsigned moe_check_word;
#define MOE_DCHECK(ok, bit)                                                   \
  do {                                                                        \
    if (!(ok)) atomicOr(&moe_check_word, (unsigned)(bit));                    \
  } while (0)
// the same, and `fix` (which makes the index safe) when the test fails
#define MOE_DCHECK_FIX(ok, bit, fix)                                          \
  do {                                                                        \
    if (!(ok)) {                                                              \
      atomicOr(&moe_check_word, (unsigned)(bit));                             \
      fix;                                                                    \
    }                                                                         \
  } while (0)
// the file's flag word, cleared after reading (the device must be idle)
#define MOE_CHECKS_READER(name)                                               \
  unsigned read_checks_##name() {                                             \
    unsigned v = 0;                                                           \
    const unsigned z = 0;                                                     \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(moe_check_word), sizeof v) != hipSuccess || \
        hipMemcpyToSymbol(HIP_SYMBOL(moe_check_word), &z, sizeof z) != hipSuccess)     \
      return ~0u;                                                             \
    return v;                                                                 \
  }
unsigned read_checks_router();
unsigned read_checks_permute();
unsigned read_checks_combine();
unsigned read_checks_gemm_persist();
unsigned read_checks_gemm_fp8();
unsigned read_checks_gemm_f32();
#else
#define MOE_DCHECK(ok, bit) \
  do {                      \
  } while (0)
#define MOE_DCHECK_FIX(ok, bit, fix) \
  do {                               \
  } while (0)
#define MOE_CHECKS_READER(name)
#endif

// ---------------------------------------------------------------- helpers
typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// float -> bfloat16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct ElemIO;
template <> struct ElemIO<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct ElemIO<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError().

// Router logits z[T, N] = x[T, d] . W_r[N, d]^T in fp32 (SIMT, fp32 FMA).
hipError_t launch_router_logits_simt(bool x_bf16, const void* x, const float* W_r, float* z,
                                     int64_t T, int d, int N, hipStream_t stream);

// Router logits on MFMA for bf16 x: W_r [N, d] split exactly into three bf16
// parts hi, mid, lo, and K split into `nsplit` partial sums
// zpart[nsplit][T][N].  With at least kRouterPresplitBlocks blocks of 128
// tokens the split is made once into `planes` ([3][N][d] bf16, workspace),
// else inside each block (planes unused, may be null).
constexpr int kRouterPresplitBlocks = 4;
bool router_presplit(int64_t T);
int router_mfma_splits(int64_t T, int d, int N);
hipError_t launch_router_logits_mfma(const bf16_t* x, const float* W_r, bf16_t* planes,
                                     float* zpart, int64_t T, int d, int N, int nsplit,
                                     hipStream_t stream);
constexpr int kRouterSelectSplits = 64;  // at most this many K splits

// Scores, group-limited top-k and gates from z (the sum of nsplit partials).
// Experts out of the selection: allow bit e of word e/64 (when `any`), then
// each token's `top` best remaining keys.
struct ExpertMask {
  uint64_t allow[4];
  int any;
  int top;
};
hipError_t launch_router_select(const float* z, int nsplit, const float* b, int64_t T, int N, int k,
                                int n_groups, int topk_groups, int group_topn, int gate,
                                float route_scale, int32_t* idx, float* gates, float* scores,
                                hipStream_t stream, const ExpertMask* mask = nullptr);
// b[i] += gamma * sign(slots - N * counts[i])
hipError_t launch_bias_update(float* b, const int32_t* counts, int N, int64_t slots, float gamma,
                              hipStream_t stream);

// Counting-sort permutation of the S = T*k slots.
constexpr int kPermChunk = 256;  // slots per wavefront chunk
constexpr int kPermIdBits = 8;   // expert ids are below 256
hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int N, int32_t* hist,
                          int32_t* base, int32_t* rank, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, hipStream_t stream);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream);
// p[0] = 0, p[1] = n: the row range of a single group covering n rows
hipError_t launch_set_range(int32_t* p, int32_t n, hipStream_t stream);
// row_token_tail[t] = t for t < T, and offsets_last[0] = end
hipError_t launch_append_shared_rows(int32_t* row_token_tail, int32_t T, int32_t* offsets_last,
                                     int32_t end, hipStream_t stream);
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, void* x_perm,
                              int64_t rows, int64_t row_bytes, hipStream_t stream);

// Grouped GEMMs.  Group g owns rows [offsets[g], offsets[g+1]); its weight
// matrix is B + g * Nout * K, stored [Nout, K].
struct GroupedGemmArgs {
  const void* A;            // activation rows [*, K]
  const int32_t* row_index; // nullable gather map
  int64_t a_rows;           // rows of A (the device checks' bound for gathered rows)
  const int32_t* offsets;   // [n_groups + 1] device
  int n_groups;
  int64_t max_rows;
  const void* B0;           // [G, Nout, K]  (W1 or W2)
  const void* B1;           // [G, Nout, K]  (W3) for the SwiGLU epilogue, else null
  const void* B0x;          // if non-null, the weights [Nout, K] of the last group (the
  const void* B1x;          //   shared expert folded in as one more group)
  const float* S0;          // fp8 block scales [G, Nout/128, K/128] or null
  const float* S1;
  const float* S0x;         // fp8: the block scales [Nout/128, K/128] of B0x / B1x
  const float* S1x;
  void* C;                  // [rows, Nout]
  int Nout;
  int K;
  const void* zero_row;     // persistent bf16 GEMMs: kZeroRows rows of K zero activations
                            //   for rows past a tile's last (null: repeat the last row)
};
constexpr int kZeroRows = 16;
// Persistent: one workgroup per CU, one pipeline across all of its tiles.
// The gathered row indices of the tile after next are read one tile after
// they were fetched, and only a tile of at least (stages) K-steps of 32 puts
// a wait and a barrier between the two: the launchers return
// hipErrorInvalidValue for a smaller K.  bf16: K >= 128 (4 stages).
hipError_t launch_gemm_bf16_persist(const GroupedGemmArgs& a, bool swiglu, hipStream_t s);
// the same with fp8 block-scaled weights, dequantized to bf16 in registers
// (K and Nout multiples of 128; 4 stages: K >= 128)
hipError_t launch_gemm_fp8_persist(const GroupedGemmArgs& a, bool swiglu, hipStream_t s);
// the smallest K each persistent kernel accepts
int persist_min_k(bool fp8_weights);
// persistent grid: one workgroup per CU of the current device, a multiple of 8
int persist_grid();
// fp32 SIMT (act f32, w f32)
hipError_t launch_gemm_f32_swiglu(const GroupedGemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f32_store(const GroupedGemmArgs& a, hipStream_t s);
// fp8 block-scaled weights, bf16 activations, small row counts (decode)
hipError_t launch_gemm_fp8_swiglu(const GroupedGemmArgs& a, hipStream_t s);
hipError_t launch_gemm_fp8_store(const GroupedGemmArgs& a, hipStream_t s);

// out = residual + y_shared + sum_j gate_j * y_perm[slot_row]
hipError_t launch_combine(bool act_bf16, bool out_bf16, const void* y_perm,
                          const int32_t* slot_row, const float* gate, const void* y_shared,
                          const void* residual, void* out, int64_t T, int d, int k,
                          hipStream_t stream);

}  // namespace moe
