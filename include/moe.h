/*
 * moe.h - C ABI of the MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * The layer (open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts",
 * "All 19 steps"; aiany.app DeepSeekMoE explainer, Steps 2, 6 and 7):
 *
 *   router   z = x W_r;  softmax p = softmax(z [+ b])      or  s = sigmoid(z)
 *            selection: top-k of the key (p, or s + b), optionally only inside
 *            the top `topk_groups` of `n_groups` expert groups
 *            gates: softmax  G = route_scale * p_sel (unrenormalised)
 *                   sigmoid  G = route_scale * s_sel / sum(s_sel)
 *   expert   E(x) = (silu(x W1) * (x W3)) W2,  silu(g) = g * sigmoid(g)
 *   layer    out = x + sum_j G_j E_{idx_j}(x) + y_shared(x)
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller, row-major
 *     and contiguous.  The library never allocates, frees or keeps a pointer
 *     after a call returns, and never synchronises the host with the device.
 *   - `stream` arguments are hipStream_t values passed as void* (NULL = the
 *     null stream).  Work is enqueued asynchronously; the caller synchronises.
 *   - Arguments are validated on the host before any launch; a failing call
 *     enqueues nothing and returns a negative moe_status.  Launch failures
 *     return MOE_ERR_HIP.  moe_last_error() gives a thread-local message.
 *   - Weights are stored output-major, the way a Linear layer stores them:
 *       W_r  [N, d]       fp32       (the router matrix d x N, transposed)
 *       W1   [E, I, d]    W3 [E, I, d]   (d x I matrices, transposed)
 *       W2   [E, d, I]                   (I x d matrix, transposed)
 *     so that every contraction reads both operands along d or I.
 *   - fp8 weights are OCP e4m3fn codes with one fp32 scale per 128 x 128 block
 *     of the stored matrix: s1, s3 [E, I/128, d/128], s2 [E, d/128, I/128].
 *   - bf16 values are passed as their 16-bit patterns.
 *   - Routing is deterministic: ties between equal keys (and between equal
 *     group scores) go to the lower index, and every reduction runs in a fixed
 *     order, so two calls with the same inputs give bitwise-equal results.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a null pointer, a bad size, k > allowed experts ... */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype mix, alignment)   */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required         */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed          */
  MOE_ERR_DEVICE_CHECK = -5 /* checked build only (libmoe_checked.so, compiled with
                               MOE_DEVICE_CHECKS=1): a kernel found an index outside
                               its range; see "Checked build" below                */
} moe_status;

/* Checked build.  The same sources compiled with MOE_DEVICE_CHECKS=1 give
 * libmoe_checked.so, a debugging aid.  There the kernels test the index
 * invariants their memory accesses rely on: top-k expert ids in [0, N), the
 * per-expert counts adding up to T*k, gathered activation rows inside the
 * activation matrix (for moe_expert_ffn with row_index: [0, T)), group
 * offsets non-negative and non-decreasing, combine slots inside the T*k
 * permuted rows, selected experts in [0, N) with finite gates.  A failed test
 * sets a bit in a device flag word (no trap) and, where the index addresses
 * memory, is replaced by a safe one.  Every entry point then synchronises the
 * device before it returns (so the checked build cannot be captured into a
 * graph) and returns MOE_ERR_DEVICE_CHECK, moe_last_error() naming the
 * failed checks.  The ordinary build compiles the checks to nothing. */

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

typedef enum {
  MOE_GATE_SOFTMAX = 0,      /* GShard / DeepSeekMoE / V2: softmax over routed experts */
  MOE_GATE_SIGMOID_NORM = 1  /* V3: sigmoid scores, selection on s+b, normalised gates */
} moe_gate_mode;

typedef struct {
  int64_t T;            /* tokens (batch x positions flattened)                        */
  int32_t d;            /* model width                                                 */
  int32_t n_routed;     /* N routed experts (1..256)                                   */
  int32_t n_shared;     /* S shared experts; they form one MLP of width S*inter        */
  int32_t inter;        /* I, intermediate width of one expert                         */
  int32_t k;            /* experts selected per token                                  */
  int32_t n_groups;     /* expert groups (1 = no group limit); must divide n_routed    */
  int32_t topk_groups;  /* groups kept per token                                       */
  int32_t group_topn;   /* keys summed into a group's score (2 for V3)                 */
  int32_t gate;         /* moe_gate_mode                                               */
  float route_scale;    /* gate scale: 2.5 for V3, 1.0 for softmax routers             */
  int32_t act_dtype;    /* x and intermediate activations: MOE_F32 or MOE_BF16         */
  int32_t w_dtype;      /* expert weights: MOE_F32, MOE_BF16 or MOE_FP8_E4M3           */
  int32_t out_dtype;    /* layer output: MOE_F32 or MOE_BF16                           */
  int32_t w_block;      /* 128 with MOE_FP8_E4M3, else 0                               */
} moe_config;

/* Supported combinations: (act, w) = (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * bf16/fp8 need d % 128 == 0 and inter % 128 == 0 (fp8: also w_block == 128);
 * f32 needs d % 64 == 0 and inter % 64 == 0. */

/* Human-readable name of a moe_status value (static string). */
const char* moe_status_string(int status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* Bytes of device workspace every entry point below may use for this config
 * (the maximum over them), or 0 if the config is invalid.  The same workspace
 * may be reused by consecutive calls on one stream. */
size_t moe_workspace_size(const moe_config* cfg);

/*
 * moe_router - router scores, group-limited top-k and gates.
 * (open-model-atlas "All 19 steps", router: z = x W_r, s = sigmoid(z),
 *  top-8 of s+b inside the top-4 groups, G = 2.5 s / sum s; aiany.app Step 2:
 *  softmax over the routed scores, the top-k probabilities are the gates.)
 *   x          [T, d]   act_dtype
 *   W_r        [N, d]   fp32
 *   b          [N]      fp32, nullable.  softmax: added to the logits before
 *                       the softmax; sigmoid: added to s for the selection only
 *   topk_idx   [T, k]   int32 out, per token ordered by key descending, index
 *                       ascending on ties
 *   topk_gate  [T, k]   fp32 out
 *   scores     [T, N]   fp32 out, nullable: p (softmax) or s (sigmoid)
 *   ws         workspace of moe_workspace_size(cfg) bytes
 */
int moe_router(const moe_config* cfg, const void* x, const float* W_r, const float* b,
               int32_t* topk_idx, float* topk_gate, float* scores,
               void* ws, size_t ws_bytes, void* stream);

/*
 * moe_router_masked - moe_router with experts taken out of the selection
 * (aiany.app explainer, Step 9, probe 1: for each token, mask the routed
 * experts the router wanted most and route among the rest; probe 2, fewer
 * picks, is moe_router with a smaller cfg->k).
 *   allow      [N] uint8 HOST array, nullable: experts with allow[e] == 0 are
 *              never selected
 *   mask_top   per token, its mask_top highest keys among the allowed experts
 *              (key descending, index ascending) are excluded as well; 0 = none
 * The scores (p or s, and so the gates of the experts that are selected) are
 * those of the unmasked router; group scores and the top-k use only the keys
 * left.  Other arguments as moe_router.  Returns MOE_ERR_INVALID_ARG unless
 * every group keeps group_topn + mask_top allowed experts and the kept groups
 * hold k + mask_top of them (so every token still finds k experts).
 */
int moe_router_masked(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                      const uint8_t* allow, int32_t mask_top, int32_t* topk_idx,
                      float* topk_gate, float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_bias_update - auxiliary-loss-free balancing step (grasp.study lesson,
 * 3.2: each expert's selection bias is nudged after a batch, up when the
 * expert was underloaded and down when it was overloaded).
 *   b          [N] fp32 device, updated in place:
 *              b[i] += gamma if N*counts[i] < T*k, -= gamma if greater, else kept
 *   counts     [N] int32 device: the batch's selections per expert (moe_permute
 *              or moe_forward's counts_out), T*k of them in total (cfg->T, cfg->k)
 *   gamma      step, finite and >= 0
 * Needs no workspace.  Enqueued on `stream`.
 */
int moe_bias_update(const moe_config* cfg, float* b, const int32_t* counts, float gamma,
                    void* stream);

/*
 * moe_permute - stable counting sort of the T*k (token, expert) slots into
 * expert-contiguous rows (the bincount and per-expert row lists of the
 * reference forward excerpt on open-model-atlas, done on the device).
 * Slot f = t*k + j.  Rows are ordered by expert, then by f.
 *   topk_idx   [T, k]   int32 in, values in [0, N).  The values are not
 *                       checked (that would need a host round trip); an id
 *                       below 0 or at or above N is treated as 0 or N-1, so
 *                       the call never reads or writes outside its buffers
 *   x          [T, d]   act_dtype, nullable (only read when x_perm != NULL)
 *   counts     [N]      int32 out: slots per expert
 *   offsets    [N+1]    int32 out: exclusive prefix sum of counts
 *   row_token  [T*k]    int32 out: token of each permuted row
 *   slot_row   [T*k]    int32 out: permuted row of each slot
 *   x_perm     [T*k, d] act_dtype out, nullable: x_perm[r] = x[row_token[r]]
 */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn - grouped SwiGLU experts over expert-contiguous rows
 * (open-model-atlas "All 19 steps", routed expert: g = x W1, u = x W3,
 *  a = g sigmoid(g), h = a * u, E = h W2).
 *   n_experts  number of experts (row groups); expert e owns rows
 *              [offsets[e], offsets[e+1]) of the row space
 *   offsets    [n_experts+1] int32 DEVICE array, non-decreasing, offsets[0]=0
 *   max_rows   host upper bound of offsets[n_experts] (sizes the launch)
 *   x_rows     activation rows, act_dtype, row length d
 *   row_index  [max_rows] int32, nullable.  NULL: row r reads x_rows[r];
 *              else row r reads x_rows[row_index[r]] (fused gather)
 *   W1, W3     [n_experts, inter, d];  W2 [n_experts, d, inter]   (w_dtype)
 *   s1, s3, s2 fp8 block scales (see above), NULL unless w_dtype is fp8
 *   y_rows     [max_rows, d] act_dtype out (rows past offsets[n] untouched)
 * The shared MLP is one expert over all T rows: n_experts = 1,
 * offsets = {0, T}, inter = n_shared * inter of the layer (cfg->inter is read
 * from `inter_override` when it is > 0).
 * Experts with no rows are never read.  fp8 weights, per projection: with at
 * least 128 rows per expert on average (max_rows >= 128 * n_experts) the
 * codes are dequantized to bf16(code * scale) for bf16
 * MFMAs (prefill); otherwise each expert's weights are streamed once, the
 * codes multiplied exactly and each 128-wide block's fp32 partial sum scaled
 * once (decode).  The two ways round differently (the first rounds every
 * dequantized weight to bf16) and both stay within the fp8 tolerance.
 */
int moe_expert_ffn(const moe_config* cfg, int32_t n_experts, const int32_t* offsets,
                   int64_t max_rows, int32_t inter_override,
                   const void* x_rows, const int32_t* row_index,
                   const void* W1, const void* W3, const void* W2,
                   const float* s1, const float* s3, const float* s2,
                   void* y_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine - deterministic gate-weighted unpermute + shared + residual
 * (open-model-atlas: y_routed = sum_i G_i E_i, Delta = y_routed + y_shared;
 *  aiany.app Step 7 and shivam2003.com "Idea 2": the layer input is added).
 *   out[t] = residual[t] + y_shared[t] + sum_{j<k} topk_gate[t,j] * y_perm[slot_row[t*k+j]]
 * summed in fp32 in exactly that order (j ascending first, then shared, then
 * residual); no atomics.
 *   y_perm     [T*k, d] act_dtype;  slot_row [T*k] int32;  topk_gate [T, k] fp32
 *   y_shared   [T, d] act_dtype, nullable (no shared experts)
 *   residual   [T, d] act_dtype, nullable (then out = Delta)
 *   out        [T, d] out_dtype
 */
int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_row,
                const float* topk_gate, const void* y_shared, const void* residual,
                void* out, void* stream);

/*
 * moe_forward - the whole layer: router -> permute -> routed experts (fused
 * gather) -> combine.  The shared MLP runs on `stream_side`, overlapping the
 * routed path: with fewer than 128 routed rows per expert (T*k < 128*N, a
 * decode step, bound by streaming weights) it starts with the router, else
 * when the routed up GEMM has ended, overlapping the routed down GEMM.
 * stream_side may be NULL or equal stream_main: then, with bf16 or fp8 weights
 * and one shared expert (S = 1), the shared expert runs inside the routed
 * grouped GEMMs as one more group whose rows are all T tokens (results are
 * bitwise the same either way), and otherwise on stream_main, before the
 * router (T*k < 128*N) or after the routed GEMMs.
 *   x [T, d];  W_r [N, d];  b [N] nullable
 *   W1, W3 [N, I, d];  W2 [N, d, I];  s1, s3, s2 fp8 scales or NULL
 *   W1s, W3s [S*I, d];  W2s [d, S*I];  s1s, s3s, s2s   (all NULL when S = 0)
 *   out [T, d] out_dtype = x + Delta
 *   topk_idx_out [T,k], topk_gate_out [T,k], counts_out [N]: nullable copies of
 *   the routing results.
 * Returns after enqueueing; stream_main carries the completion of everything.
 */
int moe_forward(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                const void* W1, const void* W3, const void* W2,
                const float* s1, const float* s3, const float* s2,
                const void* W1s, const void* W3s, const void* W2s,
                const float* s1s, const float* s3s, const float* s2s,
                void* out, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                void* ws, size_t ws_bytes, void* stream_main, void* stream_side);

/* Stages of moe_forward, in launch order (shared ones run on stream_side;
 * when the shared expert is folded into the routed GEMMs, UP and DOWN cover it
 * and the two shared stages are empty intervals on stream_main). */
typedef enum {
  MOE_STAGE_ROUTER = 0,      /* logits + selection                 (stream_main) */
  MOE_STAGE_PERMUTE = 1,     /* histogram, scan, scatter           (stream_main) */
  MOE_STAGE_UP = 2,          /* routed W1|W3 grouped GEMM + SwiGLU (stream_main) */
  MOE_STAGE_DOWN = 3,        /* routed W2 grouped GEMM             (stream_main) */
  MOE_STAGE_SHARED_UP = 4,   /* shared W1|W3 GEMM + SwiGLU         (stream_side) */
  MOE_STAGE_SHARED_DOWN = 5, /* shared W2 GEMM                     (stream_side) */
  MOE_STAGE_COMBINE = 6,     /* gate-weighted combine + residual   (stream_main) */
  MOE_NUM_STAGES = 7
} moe_stage;

/*
 * moe_forward_timed - moe_forward that also records caller-owned HIP events
 * around each stage, for measurement.  stage_events holds 2*MOE_NUM_STAGES
 * hipEvent_t values passed as void* (NULL entries are skipped): entry 2*s is
 * recorded just before stage s's first launch and entry 2*s+1 just after its
 * last, on the stream that stage runs on.  Results are identical to
 * moe_forward.
 */
int moe_forward_timed(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                      const void* W1, const void* W3, const void* W2,
                      const float* s1, const float* s3, const float* s2,
                      const void* W1s, const void* W3s, const void* W2s,
                      const float* s1s, const float* s3s, const float* s2s,
                      void* out, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                      void* ws, size_t ws_bytes, void* stream_main, void* stream_side,
                      void* const* stage_events);

/* Size of the static per-GPU scratch array of moe_forward_noalloc: 64 MiB,
 * the workspace of the V3-shaped decode step (d = 7168, 1 + 256 experts,
 * inter 2048, top-8) up to T = 256 tokens (15.2 MiB at T = 64). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * moe_forward_noalloc - moe_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as moe_forward, without
 * ws / ws_bytes: the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from its
 * first call there until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks the array's address up, and the two-stream forward's
 * fork/join events are created once per host thread and device, as in
 * moe_forward.
 *   Returns MOE_ERR_WORKSPACE, enqueueing nothing, when
 *   moe_workspace_size(cfg) > MOE_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call rewrites all it reads before reading it): calls that
 * overlap on one GPU - on different streams, or from different threads
 * without ordering between their streams - race on it.  The streams must
 * belong to the current device.
 */
int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                        const void* W1, const void* W3, const void* W2,
                        const float* s1, const float* s3, const float* s2,
                        const void* W1s, const void* W3s, const void* W2s,
                        const float* s1s, const float* s3s, const float* s2s,
                        void* out, int32_t* topk_idx_out, float* topk_gate_out,
                        int32_t* counts_out, void* stream_main, void* stream_side);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
