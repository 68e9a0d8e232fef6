// C-ABI entry points of the MI355X DeepSeekMoE layer forward: argument
// validation (pure host code, before any launch), workspace layout, and the
// orchestration of the gfx950 kernels on the caller's streams.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int status, const std::string& msg) {
  g_err = msg;
  return status;
}

#define MOE_HIP_CHECK(expr)                                                      \
  do {                                                                           \
    hipError_t e_ = (expr);                                                      \
    if (e_ != hipSuccess)                                                        \
      return fail(MOE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// The end of every entry point: in the checked build, wait for the device and
// turn the kernels' recorded check failures into MOE_ERR_DEVICE_CHECK.
int device_checks(int st) {
#if MOE_DEVICE_CHECKS
  if (st != MOE_OK) return st;
  if (hipDeviceSynchronize() != hipSuccess)
    return fail(MOE_ERR_HIP, "device checks: synchronising the device failed");
  const unsigned v = read_checks_router() | read_checks_permute() | read_checks_combine() |
                     read_checks_gemm_persist() | read_checks_gemm_fp8() | read_checks_gemm_f32();
  if (v == 0) return MOE_OK;
  if (v == ~0u) return fail(MOE_ERR_HIP, "device checks: reading the flags failed");
  std::string m = "device checks failed:";
  if (v & kCheckExpertId) m += " top-k expert id outside [0, N);";
  if (v & kCheckOffsets) m += " per-expert counts do not add up to T*k;";
  if (v & kCheckRowIndex) m += " activation row outside the activation rows;";
  if (v & kCheckGroupRows) m += " group offsets negative or decreasing;";
  if (v & kCheckSlot) m += " combine slot outside the T*k permuted rows;";
  if (v & kCheckSelect) m += " selected expert outside [0, N) or non-finite gate;";
  return fail(MOE_ERR_DEVICE_CHECK, m);
#else
  return st;
#endif
}

size_t act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }
size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
  size_t z, wplanes, idx, gate, hist, base, rank, counts, offsets, row_token, slot_row, h, y, hs,
      ys, shoff, zrow[2], total;
  int64_t h_elems;     // capacity of the h region in activation elements
  int64_t zrow_elems;  // capacity of each zero region in bf16 elements
};

// bf16 or fp8 with one shared expert and no second stream to overlap it on:
// the shared expert runs inside the routed grouped GEMMs as one more group
// (its rows: every token, in order).  The workspace is sized for both ways.
bool can_fold_shared(const moe_config& c) {
  return (c.w_dtype == MOE_BF16 || c.w_dtype == MOE_FP8_E4M3) && c.n_shared == 1;
}

Layout make_layout(const moe_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const int64_t T = c.T, N = c.n_routed, d = c.d, I = c.inter, S = c.n_shared;
  const int64_t slots = T * c.k;
  const int64_t nchunks = cdiv(slots, kPermChunk);
  const size_t as = act_bytes(c.act_dtype);
  const int64_t nsplit = c.act_dtype == MOE_BF16 ? router_mfma_splits(T, c.d, c.n_routed) : 1;
  L.z = take(nsplit * T * N * 4);
  // bf16 x: the three bf16 planes of W_r the MFMA router reads
  L.wplanes = take(c.act_dtype == MOE_BF16 && router_presplit(T) ? 3 * N * d * 2 : 0);
  L.idx = take(slots * 4);
  L.gate = take(slots * 4);
  L.hist = take(nchunks * N * 4);
  L.base = take(nchunks * N * 4);
  L.rank = take(slots * 4);
  const bool fold = can_fold_shared(c);
  const int64_t grp_rows = fold ? slots + T : slots;  // rows of the grouped GEMMs
  L.counts = take(N * 4);
  L.offsets = take((N + 2) * 4);
  L.row_token = take(grp_rows * 4);
  L.slot_row = take(slots * 4);
  const int64_t rows_max = grp_rows > T ? grp_rows : T;
  const int64_t inter_max = S * I > I ? S * I : I;
  L.h_elems = rows_max * inter_max;
  L.h = take(L.h_elems * as);
  L.y = take(grp_rows * d * as);
  L.hs = take(T * S * I * as);
  L.ys = take(S > 0 ? T * d * as : 0);
  L.shoff = take(2 * 4);
  // two regions of kZeroRows zero rows (routed GEMMs; shared expert on the
  // side stream), each row as long as the longest K of the persistent GEMMs
  L.zrow_elems = (int64_t)align_up((size_t)kZeroRows * (d > inter_max ? d : inter_max) * 2) / 2;
  L.zrow[0] = take(L.zrow_elems * 2);
  L.zrow[1] = take(L.zrow_elems * 2);
  L.total = off;
  return L;
}

int check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (c->d <= 0 || c->inter <= 0) return fail(MOE_ERR_INVALID_ARG, "d and inter must be > 0");
  if (c->n_routed < 1 || c->n_routed > 256)
    return fail(MOE_ERR_UNSUPPORTED, "n_routed must be in [1, 256]");
  if (c->k < 1 || c->k > c->n_routed) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, n_routed]");
  if (c->k > 64) return fail(MOE_ERR_UNSUPPORTED, "k must be <= 64");
  if (c->n_groups < 1 || c->n_groups > 64 || c->n_routed % c->n_groups != 0)
    return fail(MOE_ERR_INVALID_ARG, "n_groups must be in [1, 64] and divide n_routed");
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups)
    return fail(MOE_ERR_INVALID_ARG, "topk_groups must be in [1, n_groups]");
  const int gs = c->n_routed / c->n_groups;
  if (c->n_groups > 1 && (c->group_topn < 1 || c->group_topn > gs))
    return fail(MOE_ERR_INVALID_ARG, "group_topn must be in [1, n_routed / n_groups]");
  if ((int64_t)c->k > (int64_t)c->topk_groups * gs)
    return fail(MOE_ERR_INVALID_ARG, "k exceeds the experts of the kept groups");
  if (c->gate != MOE_GATE_SOFTMAX && c->gate != MOE_GATE_SIGMOID_NORM)
    return fail(MOE_ERR_INVALID_ARG, "unknown gate mode");
  if (!std::isfinite(c->route_scale)) return fail(MOE_ERR_INVALID_ARG, "route_scale not finite");
  if (c->n_shared < 0) return fail(MOE_ERR_INVALID_ARG, "n_shared must be >= 0");
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "out_dtype must be F32 or BF16");
  const bool f32 = c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32 && c->w_block == 0;
  const bool bf16 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_BF16 && c->w_block == 0;
  const bool fp8 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_FP8_E4M3 && c->w_block == 128;
  if (!(f32 || bf16 || fp8))
    return fail(MOE_ERR_UNSUPPORTED,
                "supported (act, w, w_block): (F32, F32, 0), (BF16, BF16, 0), (BF16, FP8_E4M3, 128)");
  const int q = f32 ? 64 : 128;
  if (c->d % q != 0 || c->inter % q != 0)
    return fail(MOE_ERR_UNSUPPORTED, f32 ? "f32 path needs d % 64 == 0 and inter % 64 == 0"
                                         : "bf16/fp8 paths need d % 128 == 0 and inter % 128 == 0");
  if (c->T * (int64_t)c->k > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "T * k must fit int32");
  return MOE_OK;
}

int check_ws(const moe_config* c, void* ws, size_t ws_bytes) {
  const size_t need = make_layout(*c).total;
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required, got " +
                                       std::to_string(ws ? ws_bytes : 0));
  return MOE_OK;
}

// The fork and join events of the two-stream forward: created once per host
// thread and device on first use and kept for the life of the thread (a
// thread enqueues one forward at a time, and a stream wait takes the event's
// state at the time of the call, so reuse by the thread's next forward is
// safe; per thread, so concurrent callers never share them).
int fork_join_events(hipEvent_t* fork, hipEvent_t* join) {
  constexpr int kMaxDev = 64;
  thread_local hipEvent_t ev[kMaxDev][2] = {};
  int dev = 0;
  MOE_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDev) return fail(MOE_ERR_UNSUPPORTED, "device ordinal above 63");
  for (int i = 0; i < 2; ++i)
    if (!ev[dev][i]) MOE_HIP_CHECK(hipEventCreateWithFlags(&ev[dev][i], hipEventDisableTiming));
  *fork = ev[dev][0];
  *join = ev[dev][1];
  return MOE_OK;
}

// Stage boundaries of the forward: a roctx range per stage on the host (seen
// by rocprofv3 --marker-trace; host-side only, so graph capture records
// nothing of them), and stage event 2*stage (+1 for the end) when the caller
// supplied it.  A range is left open only when a launch fails in between.
const char* const kStageNames[MOE_NUM_STAGES] = {"moe router", "moe permute", "moe routed up",
                                                 "moe routed down", "moe shared up",
                                                 "moe shared down", "moe combine"};

hipError_t mark(void* const* ev, int stage, bool end, hipStream_t s) {
  if (stage < 0) return hipSuccess;
  if (end) roctxRangePop();
  else roctxRangePushA(kStageNames[stage]);
  if (!ev) return hipSuccess;
  void* e = ev[2 * stage + (end ? 1 : 0)];
  return e ? hipEventRecord((hipEvent_t)e, s) : hipSuccess;
}

// The roctx range of one whole forward, closed on every return path.
struct ForwardRange {
  ForwardRange() { roctxRangePushA("moe_forward"); }
  ~ForwardRange() { roctxRangePop(); }
};

template <typename P>
P* at(void* ws, size_t off) {
  return (P*)((char*)ws + off);
}

int run_router(const moe_config* c, const void* x, const float* W_r, const float* b,
               int32_t* idx, float* gate, float* scores, void* ws, hipStream_t s,
               const ExpertMask* mask = nullptr) {
  const Layout L = make_layout(*c);
  float* z = at<float>(ws, L.z);
  int nsplit = 1;
  if (c->act_dtype == MOE_BF16) {
    nsplit = router_mfma_splits(c->T, c->d, c->n_routed);
    MOE_HIP_CHECK(launch_router_logits_mfma((const bf16_t*)x, W_r, at<bf16_t>(ws, L.wplanes), z,
                                            c->T, c->d, c->n_routed, nsplit, s));
  } else {
    MOE_HIP_CHECK(launch_router_logits_simt(false, x, W_r, z, c->T, c->d, c->n_routed, s));
  }
  MOE_HIP_CHECK(launch_router_select(z, nsplit, b, c->T, c->n_routed, c->k, c->n_groups, c->topk_groups,
                                     c->group_topn, c->gate, c->route_scale, idx, gate, scores, s,
                                     mask));
  return MOE_OK;
}

// Host check that every token still finds k experts after the exclusions:
// every group keeps group_topn + mask_top allowed experts and the kept groups
// hold k + mask_top of them.
int build_mask(const moe_config* c, const uint8_t* allow, int32_t mask_top, ExpertMask* m) {
  *m = ExpertMask{};
  if (mask_top < 0) return fail(MOE_ERR_INVALID_ARG, "mask_top must be >= 0");
  const int N = c->n_routed, G = c->n_groups, gs = N / G;
  int min_group = gs;
  for (int g = 0; g < G; ++g) {
    int n = 0;
    for (int e = g * gs; e < (g + 1) * gs; ++e)
      if (!allow || allow[e]) {
        ++n;
        m->allow[e >> 6] |= 1ull << (e & 63);
      }
    min_group = n < min_group ? n : min_group;
  }
  m->any = allow ? 1 : 0;
  m->top = mask_top;
  if (G > 1 && min_group < c->group_topn + mask_top)
    return fail(MOE_ERR_INVALID_ARG,
                "every group must keep group_topn + mask_top allowed experts");
  if ((int64_t)min_group * (G > 1 ? c->topk_groups : 1) < (int64_t)c->k + mask_top)
    return fail(MOE_ERR_INVALID_ARG, "fewer than k experts would remain after the exclusions");
  return MOE_OK;
}

int run_expert_ffn(const moe_config* c, int n_experts, const int32_t* offsets, int64_t max_rows,
                   int inter, const void* x_rows, const int32_t* row_index, const void* W1,
                   const void* W3, const void* W2, const float* s1, const float* s3,
                   const float* s2, void* h, void* y_rows, hipStream_t s,
                   void* const* ev = nullptr, int stage_up = -1, int stage_dn = -1,
                   const void* W1x = nullptr, const void* W3x = nullptr,
                   const void* W2x = nullptr, const float* s1x = nullptr,
                   const float* s3x = nullptr, const float* s2x = nullptr,
                   void* zrow = nullptr, int64_t zrow_elems = 0, hipEvent_t after_up = nullptr) {
  GroupedGemmArgs up{};
  up.B0x = W1x;
  up.B1x = W3x;
  up.S0x = s1x;
  up.S1x = s3x;
  up.A = x_rows;
  up.row_index = row_index;
  up.a_rows = row_index ? c->T : max_rows;
  up.offsets = offsets;
  up.n_groups = n_experts;
  up.max_rows = max_rows;
  up.B0 = W1;
  up.B1 = W3;
  up.S0 = s1;
  up.S1 = s3;
  up.C = h;
  up.Nout = inter;
  up.K = c->d;
  GroupedGemmArgs dn{};
  dn.B0x = W2x;
  dn.S0x = s2x;
  dn.A = h;
  dn.row_index = nullptr;
  dn.a_rows = max_rows;
  dn.offsets = offsets;
  dn.n_groups = n_experts;
  dn.max_rows = max_rows;
  dn.B0 = W2;
  dn.B1 = nullptr;
  dn.S0 = s2;
  dn.S1 = nullptr;
  dn.C = y_rows;
  dn.Nout = c->d;
  dn.K = inter;
  // bf16: the persistent MFMA kernel (K is a multiple of 128, so at least
  // the four 32-deep steps its pipeline has stages for).  fp8: many rows per
  // expert (prefill) take the same kernel with the weights dequantized to
  // bf16 in registers (its four stages need K >= 128, which every fp8 config
  // has); a few rows per expert (decode), the weight-streaming kernel, which
  // takes any row count.
  auto persistent = [&](const GroupedGemmArgs& a) {
    if (c->w_dtype == MOE_BF16) return true;
    return c->w_dtype == MOE_FP8_E4M3 && a.max_rows >= 128 * (int64_t)a.n_groups &&
           a.K >= persist_min_k(true);
  };
  // the persistent kernels' rows past a tile's last read a row of zeros
  // (same results, less power than repeating the last row): cleared here
  const int64_t kmax = c->d > inter ? c->d : inter;
  if (zrow && zrow_elems >= kZeroRows * kmax && (persistent(up) || persistent(dn))) {
    MOE_HIP_CHECK(launch_fill_i32((int32_t*)zrow, kZeroRows * kmax / 2, 0, s));
    up.zero_row = zrow;
    dn.zero_row = zrow;
  }
  auto fp8_gemm = [&](const GroupedGemmArgs& a, bool swiglu) {
    if (persistent(a)) return launch_gemm_fp8_persist(a, swiglu, s);
    return swiglu ? launch_gemm_fp8_swiglu(a, s) : launch_gemm_fp8_store(a, s);
  };
  MOE_HIP_CHECK(mark(ev, stage_up, false, s));
  if (c->w_dtype == MOE_F32)
    MOE_HIP_CHECK(launch_gemm_f32_swiglu(up, s));
  else if (c->w_dtype == MOE_BF16)
    MOE_HIP_CHECK(launch_gemm_bf16_persist(up, true, s));
  else
    MOE_HIP_CHECK(fp8_gemm(up, true));
  MOE_HIP_CHECK(mark(ev, stage_up, true, s));
  if (after_up) MOE_HIP_CHECK(hipEventRecord(after_up, s));
  MOE_HIP_CHECK(mark(ev, stage_dn, false, s));
  if (c->w_dtype == MOE_F32)
    MOE_HIP_CHECK(launch_gemm_f32_store(dn, s));
  else if (c->w_dtype == MOE_BF16)
    MOE_HIP_CHECK(launch_gemm_bf16_persist(dn, false, s));
  else
    MOE_HIP_CHECK(fp8_gemm(dn, false));
  MOE_HIP_CHECK(mark(ev, stage_dn, true, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE_CHECK: return "MOE_ERR_DEVICE_CHECK";
    default: return "MOE_UNKNOWN_STATUS";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return make_layout(*cfg).total;
}

int moe_router(const moe_config* cfg, const void* x, const float* W_r, const float* b,
               int32_t* topk_idx, float* topk_gate, float* scores, void* ws, size_t ws_bytes,
               void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !W_r || !topk_idx || !topk_gate)
    return fail(MOE_ERR_INVALID_ARG, "x, W_r, topk_idx and topk_gate must be non-NULL");
  if ((st = check_ws(cfg, ws, ws_bytes))) return st;
  return device_checks(
      run_router(cfg, x, W_r, b, topk_idx, topk_gate, scores, ws, (hipStream_t)stream));
}

int moe_router_masked(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                      const uint8_t* allow, int32_t mask_top, int32_t* topk_idx, float* topk_gate,
                      float* scores, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  ExpertMask m;
  if ((st = build_mask(cfg, allow, mask_top, &m))) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !W_r || !topk_idx || !topk_gate)
    return fail(MOE_ERR_INVALID_ARG, "x, W_r, topk_idx and topk_gate must be non-NULL");
  if ((st = check_ws(cfg, ws, ws_bytes))) return st;
  return device_checks(
      run_router(cfg, x, W_r, b, topk_idx, topk_gate, scores, ws, (hipStream_t)stream, &m));
}

int moe_bias_update(const moe_config* cfg, float* b, const int32_t* counts, float gamma,
                    void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  if (!b || !counts) return fail(MOE_ERR_INVALID_ARG, "b and counts must be non-NULL");
  if (!std::isfinite(gamma) || gamma < 0.f)
    return fail(MOE_ERR_INVALID_ARG, "gamma must be finite and >= 0");
  MOE_HIP_CHECK(launch_bias_update(b, counts, cfg->n_routed, cfg->T * (int64_t)cfg->k, gamma,
                                   (hipStream_t)stream));
  return device_checks(MOE_OK);
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm, void* ws,
                size_t ws_bytes, void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts and offsets must be non-NULL");
  if (cfg->T > 0 && (!topk_idx || !row_token || !slot_row))
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, row_token and slot_row must be non-NULL");
  if (x_perm && !x) return fail(MOE_ERR_INVALID_ARG, "x_perm needs x");
  if ((st = check_ws(cfg, ws, ws_bytes))) return st;
  hipStream_t s = (hipStream_t)stream;
  const Layout L = make_layout(*cfg);
  if (cfg->T == 0) {
    MOE_HIP_CHECK(launch_fill_i32(counts, cfg->n_routed, 0, s));
    MOE_HIP_CHECK(launch_fill_i32(offsets, cfg->n_routed + 1, 0, s));
    return MOE_OK;
  }
  MOE_HIP_CHECK(launch_permute(topk_idx, cfg->T, cfg->k, cfg->n_routed, at<int32_t>(ws, L.hist),
                               at<int32_t>(ws, L.base), at<int32_t>(ws, L.rank), counts, offsets,
                               row_token, slot_row, s));
  if (x_perm)
    MOE_HIP_CHECK(launch_gather_rows(x, row_token, x_perm, cfg->T * cfg->k,
                                     (int64_t)cfg->d * act_bytes(cfg->act_dtype), s));
  return device_checks(MOE_OK);
}

int moe_expert_ffn(const moe_config* cfg, int32_t n_experts, const int32_t* offsets,
                   int64_t max_rows, int32_t inter_override, const void* x_rows,
                   const int32_t* row_index, const void* W1, const void* W3, const void* W2,
                   const float* s1, const float* s3, const float* s2, void* y_rows, void* ws,
                   size_t ws_bytes, void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  if (n_experts < 1 || n_experts > 256)
    return fail(MOE_ERR_INVALID_ARG, "n_experts must be in [1, 256]");
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "max_rows must be >= 0");
  if (max_rows == 0) return MOE_OK;
  if (!offsets || !x_rows || !W1 || !W3 || !W2 || !y_rows)
    return fail(MOE_ERR_INVALID_ARG, "offsets, x_rows, W1, W3, W2 and y_rows must be non-NULL");
  const bool fp8 = cfg->w_dtype == MOE_FP8_E4M3;
  if (fp8 && (!s1 || !s3 || !s2)) return fail(MOE_ERR_INVALID_ARG, "fp8 weights need s1, s3, s2");
  if (!fp8 && (s1 || s3 || s2)) return fail(MOE_ERR_INVALID_ARG, "scales given for non-fp8 weights");
  const int inter = inter_override > 0 ? inter_override : cfg->inter;
  const int q = cfg->w_dtype == MOE_F32 ? 64 : 128;
  if (inter % q != 0) return fail(MOE_ERR_UNSUPPORTED, "inter_override must be a multiple of 64/128");
  if ((st = check_ws(cfg, ws, ws_bytes))) return st;
  const Layout L = make_layout(*cfg);
  if (max_rows * (int64_t)inter > L.h_elems)
    return fail(MOE_ERR_WORKSPACE, "max_rows * inter exceeds the workspace sized for this config");
  if (max_rows > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "max_rows must fit int32");
  return device_checks(run_expert_ffn(
      cfg, n_experts, offsets, max_rows, inter, x_rows, row_index, W1, W3, W2, s1, s3, s2,
      at<void>(ws, L.h), y_rows, (hipStream_t)stream, nullptr, -1, -1, nullptr, nullptr, nullptr,
      nullptr, nullptr, nullptr, at<void>(ws, L.zrow[0]), L.zrow_elems));
}

int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_row,
                const float* topk_gate, const void* y_shared, const void* residual, void* out,
                void* stream) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!y_perm || !slot_row || !topk_gate || !out)
    return fail(MOE_ERR_INVALID_ARG, "y_perm, slot_row, topk_gate and out must be non-NULL");
  MOE_HIP_CHECK(launch_combine(cfg->act_dtype == MOE_BF16, cfg->out_dtype == MOE_BF16, y_perm,
                               slot_row, topk_gate, y_shared, residual, out, cfg->T, cfg->d,
                               cfg->k, (hipStream_t)stream));
  return device_checks(MOE_OK);
}

static int forward_impl(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                        const void* W1, const void* W3, const void* W2, const float* s1,
                        const float* s3, const float* s2, const void* W1s, const void* W3s,
                        const void* W2s, const float* s1s, const float* s3s, const float* s2s,
                        void* out, int32_t* topk_idx_out, float* topk_gate_out,
                        int32_t* counts_out, void* ws, size_t ws_bytes, void* stream_main,
                        void* stream_side, void* const* ev) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  const moe_config& c = *cfg;
  if (c.T == 0) {
    if (counts_out) MOE_HIP_CHECK(launch_fill_i32(counts_out, c.n_routed, 0, (hipStream_t)stream_main));
    return MOE_OK;
  }
  if (!x || !W_r || !W1 || !W3 || !W2 || !out)
    return fail(MOE_ERR_INVALID_ARG, "x, W_r, W1, W3, W2 and out must be non-NULL");
  const bool fp8 = c.w_dtype == MOE_FP8_E4M3;
  if (fp8 && (!s1 || !s3 || !s2)) return fail(MOE_ERR_INVALID_ARG, "fp8 weights need s1, s3, s2");
  if (c.n_shared > 0) {
    if (!W1s || !W3s || !W2s) return fail(MOE_ERR_INVALID_ARG, "shared weights must be non-NULL");
    if (fp8 && (!s1s || !s3s || !s2s))
      return fail(MOE_ERR_INVALID_ARG, "fp8 shared weights need s1s, s3s, s2s");
  }
  if ((st = check_ws(cfg, ws, ws_bytes))) return st;
  const ForwardRange range;
  const Layout L = make_layout(c);
  hipStream_t sm = (hipStream_t)stream_main;
  hipStream_t ss = stream_side ? (hipStream_t)stream_side : sm;
  const bool fold = can_fold_shared(c) && ss == sm;
  const bool two_streams = ss != sm && c.n_shared > 0;

  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // Where the shared expert starts on the side stream.  Few rows per routed
  // expert (decode): with the router, whose phase leaves HBM idle, the
  // layer being bound by streaming weights.  Many (prefill): when the routed
  // up projection has ended, overlapping the routed down projection; the
  // routed up GEMM then runs alone, and the forward takes as long as when the
  // shared expert starts with the router.
  const bool fork_early = c.T * (int64_t)c.k < 128 * (int64_t)c.n_routed;
  if (two_streams && (st = fork_join_events(&ev_fork, &ev_join))) return st;
  void* ys = nullptr;
  // shared MLP of width S * I over every token (one expert, rows {0, T})
  auto run_shared = [&]() -> int {
    if (two_streams) MOE_HIP_CHECK(hipStreamWaitEvent(ss, ev_fork, 0));
    int32_t* shoff = at<int32_t>(ws, L.shoff);
    ys = at<void>(ws, L.ys);
    MOE_HIP_CHECK(launch_set_range(shoff, (int32_t)c.T, ss));
    const int r = run_expert_ffn(cfg, 1, shoff, c.T, c.n_shared * c.inter, x, nullptr, W1s, W3s,
                                 W2s, s1s, s3s, s2s, at<void>(ws, L.hs), ys, ss, ev,
                                 MOE_STAGE_SHARED_UP, MOE_STAGE_SHARED_DOWN, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, at<void>(ws, L.zrow[1]),
                                 L.zrow_elems);
    if (r) return r;
    if (two_streams) MOE_HIP_CHECK(hipEventRecord(ev_join, ss));
    return MOE_OK;
  };
  const bool shared_side = c.n_shared > 0 && !fold;
  if (shared_side && fork_early) {
    if (two_streams) MOE_HIP_CHECK(hipEventRecord(ev_fork, sm));
    if ((st = run_shared())) return st;
  }
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
  float* gate = topk_gate_out ? topk_gate_out : at<float>(ws, L.gate);
  int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_ROUTER, false, sm));
  if ((st = run_router(cfg, x, W_r, b, idx, gate, nullptr, ws, sm))) return st;
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_ROUTER, true, sm));
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_PERMUTE, false, sm));
  MOE_HIP_CHECK(launch_permute(idx, c.T, c.k, c.n_routed, at<int32_t>(ws, L.hist),
                               at<int32_t>(ws, L.base), at<int32_t>(ws, L.rank), counts, offsets,
                               row_token, slot_row, sm));
  const int64_t slots = c.T * c.k;
  if (fold)
    MOE_HIP_CHECK(launch_append_shared_rows(row_token + slots, (int32_t)c.T,
                                            offsets + c.n_routed + 1, (int32_t)(slots + c.T), sm));
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_PERMUTE, true, sm));
  void* y = at<void>(ws, L.y);
  if (fold) {
    // routed experts and the shared expert (group n_routed) in one launch each
    st = run_expert_ffn(cfg, c.n_routed + 1, offsets, slots + c.T, c.inter, x, row_token, W1, W3,
                        W2, s1, s3, s2, at<void>(ws, L.h), y, sm, ev, MOE_STAGE_UP,
                        MOE_STAGE_DOWN, W1s, W3s, W2s, s1s, s3s, s2s, at<void>(ws, L.zrow[0]),
                        L.zrow_elems);
    ys = (char*)y + slots * c.d * act_bytes(c.act_dtype);
    for (int stg : {MOE_STAGE_SHARED_UP, MOE_STAGE_SHARED_DOWN}) {  // folded: empty intervals
      MOE_HIP_CHECK(mark(ev, stg, false, sm));
      MOE_HIP_CHECK(mark(ev, stg, true, sm));
    }
  } else {
    st = run_expert_ffn(cfg, c.n_routed, offsets, slots, c.inter, x, row_token, W1, W3, W2, s1,
                        s3, s2, at<void>(ws, L.h), y, sm, ev, MOE_STAGE_UP, MOE_STAGE_DOWN, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, at<void>(ws, L.zrow[0]),
                        L.zrow_elems, two_streams && !fork_early ? ev_fork : nullptr);
  }
  if (st) return st;
  if (shared_side && !fork_early && (st = run_shared())) return st;
  if (two_streams) MOE_HIP_CHECK(hipStreamWaitEvent(sm, ev_join, 0));
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_COMBINE, false, sm));
  MOE_HIP_CHECK(launch_combine(c.act_dtype == MOE_BF16, c.out_dtype == MOE_BF16, y, slot_row, gate,
                               ys, x, out, c.T, c.d, c.k, sm));
  MOE_HIP_CHECK(mark(ev, MOE_STAGE_COMBINE, true, sm));
  return MOE_OK;
}

int moe_forward(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                const void* W1, const void* W3, const void* W2, const float* s1, const float* s3,
                const float* s2, const void* W1s, const void* W3s, const void* W2s,
                const float* s1s, const float* s3s, const float* s2s, void* out,
                int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out, void* ws,
                size_t ws_bytes, void* stream_main, void* stream_side) {
  return device_checks(forward_impl(cfg, x, W_r, b, W1, W3, W2, s1, s3, s2, W1s, W3s, W2s, s1s,
                                    s3s, s2s, out, topk_idx_out, topk_gate_out, counts_out, ws,
                                    ws_bytes, stream_main, stream_side, nullptr));
}

int moe_forward_timed(const moe_config* cfg, const void* x, const float* W_r, const float* b,
                      const void* W1, const void* W3, const void* W2, const float* s1,
                      const float* s3, const float* s2, const void* W1s, const void* W3s,
                      const void* W2s, const float* s1s, const float* s3s, const float* s2s,
                      void* out, int32_t* topk_idx_out, float* topk_gate_out,
                      int32_t* counts_out, void* ws, size_t ws_bytes, void* stream_main,
                      void* stream_side, void* const* stage_events) {
  return device_checks(forward_impl(cfg, x, W_r, b, W1, W3, W2, s1, s3, s2, W1s, W3s, W2s, s1s,
                                    s3s, s2s, out, topk_idx_out, topk_gate_out, counts_out, ws,
                                    ws_bytes, stream_main, stream_side, stage_events));
}

}  // extern "C"

// ---------------------------------------------------------------- no allocation
// The forward for callers that cannot allocate: its workspace is this static
// array, one copy per GPU, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDev = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDev];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up on the first call there.
int scratch_for_current_device(void** out) {
  int dev = 0;
  MOE_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDev) return fail(MOE_ERR_UNSUPPORTED, "device ordinal above 63");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      MOE_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* W_r,
                                   const float* b, const void* W1, const void* W3, const void* W2,
                                   const float* s1, const float* s3, const float* s2,
                                   const void* W1s, const void* W3s, const void* W2s,
                                   const float* s1s, const float* s3s, const float* s2s, void* out,
                                   int32_t* topk_idx_out, float* topk_gate_out,
                                   int32_t* counts_out, void* stream_main, void* stream_side) {
  g_err.clear();
  int st = check_config(cfg);
  if (st) return st;
  const size_t need = make_layout(*cfg).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "this config needs " + std::to_string(need) +
                                       " bytes of workspace; moe_forward_noalloc has " +
                                       std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) +
                                       " (use moe_forward with a workspace)");
  void* ws = nullptr;
  if (cfg->T > 0 && (st = scratch_for_current_device(&ws))) return st;
  return device_checks(forward_impl(cfg, x, W_r, b, W1, W3, W2, s1, s3, s2, W1s, W3s, W2s, s1s,
                                    s3s, s2s, out, topk_idx_out, topk_gate_out, counts_out, ws,
                                    MOE_NOALLOC_SCRATCH_BYTES, stream_main, stream_side,
                                    nullptr));
}
