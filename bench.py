"""Benchmark of the MI355X DeepSeekMoE layer forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_prefill]

A step is one whole layer forward (router -> permute -> routed experts ->
shared expert on a second stream -> combine) over one batch of seeded
synthetic inputs already resident in HBM.  Prints one JSON line:

* value: tokens/s of the V3-shaped prefill (T=16384, d=7168, 1 shared + 256
  routed experts, top-8 in the top-4 of 8 groups, bf16);
* roofline: the dominant kernel (the routed W1|W3 grouped GEMM + SwiGLU),
  timed with HIP events recorded by the library around its launch on the
  stream it runs on, against the bf16 MFMA peak;
* decode: the fp8 decode step (T=64) as HBM GB/s over the weights of the
  experts that receive tokens, and its dominant kernel's roofline;
* configs: the GShard (fp32), DeepSeekMoE and V2-shaped layers, each with
  tokens/s and the layer's fraction of the MFMA peak;
* cpu_baseline: the fp64 oracle on the host cores over a bounded sample;
* parity (per workload, from the same CPU leg): the oracle's routing of all
  tokens against the GPU's (near ties counted), and the output of the first
  rows against the oracle's, relative to the RMS of the oracle's output.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA, MI355X
PEAK_HBM_GBPS = 8000.0     # HBM3E
STAGES = ["router", "permute", "up", "down", "shared_up", "shared_down", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the HIP runtime torch already loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixture_experts_ffn_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "routed_up_gemm_v3_prefill_v3_decode_pmc_traffic.txt")
COPY_CAL_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes


def read_traffic_db():
    """The JSON object in the PMC traffic summary (lines after the '#' header)."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    with open(TRAFFIC_FILE) as f:
        body = "".join(l for l in f if not l.startswith("#"))
    return json.loads(body) if body.strip() else {}


def traffic_from_profile(kernel_key: str, sources, algorithmic_per_launch):
    """HBM bytes per launch from the committed PMC summary, or None when the
    kernel's sources changed since the counters were taken."""
    db = read_traffic_db()
    ent = db.get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest(*sources):
        return None
    return ent.get("hbm_bytes_per_launch")


def time_next_rows(moe, c, dev, counts, events: HipEvents, stream, reps=20):
    """Event-timed averages on the workload's own inputs: the router alone, the
    router with each token's favourite expert masked (probe 1), and the
    aux-loss-free bias step on the forward's counts."""
    import torch
    b = dev["b"] if dev["b"] is not None else torch.zeros(c.n_routed, device="cuda")
    b = b.clone()
    calls = {
        "router_ms": lambda: moe.router(c, dev["x"], dev["w_r"], b),
        "router_mask_top1_ms": lambda: moe.router_masked(c, dev["x"], dev["w_r"], b, mask_top=1),
        "bias_update_ms": lambda: moe.bias_update(c, b, counts, 1e-3),
    }
    out = {}
    for name, fn in calls.items():
        e0, e1 = events.create(2)
        t_w = time.perf_counter()
        n_w = 0
        while time.perf_counter() - t_w < 0.1:  # back-to-back calls first (clocks)
            fn()
            n_w += 1
            if n_w % 16 == 0:
                torch.cuda.synchronize()
        rec = events.hip.hipEventRecord
        rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rec(e0, stream.cuda_stream)
        for _ in range(reps):
            fn()
        rec(e1, stream.cuda_stream)
        torch.cuda.synchronize()
        out[name] = round(events.elapsed_ms(e0, e1) / reps, 4)
        events.destroy([e0, e1])
    return out


WARM_S = 0.5  # seconds of back-to-back forwards before the timed ones
RESTAGE_S = 0.25  # seconds of eager forwards before the stage-event ones


def gpu_sclk_mhz():
    """The GPU's current shader clock in MHz: the level marked current in the
    driver's sysfs table (the file rocm-smi reads), or None if there is not
    exactly one such GPU.  A plain file read: no child process."""
    import glob
    found = []
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        found.append(int(line.split(":")[1].strip().lower().split("mhz")[0]))
        except (OSError, ValueError, IndexError):
            continue
    return found[0] if len(found) == 1 else None


def shared_placement(cfg, two_streams: bool) -> str:
    """How the timed forward runs the shared expert: folded into the routed
    grouped GEMMs as one more group (one stream; bf16 or fp8 weights and one
    shared expert), else on a second stream."""
    if not two_streams and cfg.n_shared == 1 and cfg.w_dtype in ("bf16", "fp8"):
        return "folded"
    return "side stream" if cfg.n_shared > 0 else "none"


def run_workload(name, steps, warmup, events: HipEvents, extra=False, two_streams=False,
                 overrides=None, graph=True, check_rows=48):
    import torch
    import datagen
    from datagen.device import upload
    import mixture_experts_ffn_gemm_amd as moe

    cfg = datagen.get_config(name, **(overrides or {}))
    t0 = time.time()
    inp = datagen.MoEInputs(cfg)
    dev = upload(inp)
    log(f"[bench] {name}: inputs generated and resident in {time.time() - t0:.1f}s")
    c = moe.config_from(cfg)
    ws = moe.Workspace.get(c, "cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.n_routed, dtype=torch.int32, device="cuda")
    main = torch.cuda.current_stream()
    placement = shared_placement(cfg, two_streams)
    one_stream = placement == "folded"
    side = main if one_stream else torch.cuda.Stream()
    L = moe._lib.LIB
    ex, sh = dev["experts"], dev["shared"] or {}
    P = lambda t: None if t is None else t.data_ptr()
    ev_arr_t = ctypes.c_void_p * (2 * len(STAGES))
    n_ev = 2 * len(STAGES) * steps
    evs = events.create(n_ev)

    def step(ev_ptr, stream=main):
        st = L.moe_forward_timed(
            c, P(dev["x"]), P(dev["w_r"]), P(dev["b"]), P(ex["w1"]), P(ex["w3"]), P(ex["w2"]),
            P(ex.get("s1")), P(ex.get("s3")), P(ex.get("s2")), P(sh.get("w1")), P(sh.get("w3")),
            P(sh.get("w2")), P(sh.get("s1")), P(sh.get("s3")), P(sh.get("s2")), out.data_ptr(),
            None, None, counts.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream,
            (stream if one_stream else side).cuda_stream, ev_ptr)
        if st != 0:
            raise RuntimeError(f"moe_forward_timed: {moe.status_string(st)}: {moe.last_error()}")

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    run = lambda: step(None)
    if graph:
        # one forward (both streams) captured in a HIP graph, replayed per step
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(main)
        with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
            step(None, cap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        run = g.replay
    # Sustained-load warm-up before the timed steps: at least `warmup` more
    # forwards and at least WARM_S seconds of back-to-back ones, and no idle
    # gap between it and the timed steps.  After an idle gap (graph capture,
    # a host call of a few hundred ms) replayed decode forwards slow from 1.20
    # to 1.41 ms and settle at 1.13 ms only after about 15 of them, prefill
    # forwards take 16.8 and 15.1 ms before settling at 14.5 ms (clocks
    # adjusting to the load); a fixed count of a few steps does not cover it.
    sclk0 = gpu_sclk_mhz()  # before the warm-up: an idle gap after it slows the next steps
    tev = events.create(steps + 1)
    rec = events.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    t_w = time.perf_counter()
    n_w = 0
    while n_w < warmup or time.perf_counter() - t_w < WARM_S:
        run()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()  # keep the host's clock on the GPU's
    torch.cuda.synchronize()
    # the timed steps carry no stage events (the per-stage times come from as
    # many eager steps again, each stage bracketed by events on its own
    # stream), only one event after each step on the stream the steps run on,
    # for the per-step median and spread (the host clock gives the total)
    t_start = time.perf_counter()
    rec(tev[0], main.cuda_stream)
    for i in range(steps):
        run()
        rec(tev[i + 1], main.cuda_stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # the stage-event steps follow at once, after RESTAGE_S more seconds of
    # eager forwards, so that they too run at the clocks of sustained load
    arrays = [ev_arr_t(*evs[i * 2 * len(STAGES):(i + 1) * 2 * len(STAGES)]) for i in range(steps)]
    t_w = time.perf_counter()
    n_w = 0
    while time.perf_counter() - t_w < RESTAGE_S:
        step(None)
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    for i in range(steps):
        step(arrays[i])
    torch.cuda.synchronize()
    sclk1 = gpu_sclk_mhz()
    in_order = [events.elapsed_ms(tev[i], tev[i + 1]) for i in range(steps)]
    per_step = sorted(in_order)
    events.destroy(tev)
    spread = {"median_ms": round(per_step[len(per_step) // 2] if steps % 2 else
                                 0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2]), 4),
              "min_ms": round(per_step[0], 4), "max_ms": round(per_step[-1], 4),
              "sclk_mhz": {"before_warmup": sclk0, "after_stage_steps": sclk1}}
    stage_ms = {s: [] for s in STAGES}
    for i in range(steps):
        base = i * 2 * len(STAGES)
        for j, s in enumerate(STAGES):
            if s.startswith("shared") and cfg.n_shared == 0:
                continue
            stage_ms[s].append(events.elapsed_ms(evs[base + 2 * j], evs[base + 2 * j + 1]))
    events.destroy(evs)
    avg = {s: (sum(v) / len(v) if v else 0.0) for s, v in stage_ms.items()}
    counts_np = counts.cpu().numpy()
    # the routing and the first rows of one more forward (same launch shape),
    # for the CPU leg's comparison with the oracle
    o2, idx2, gate2, counts2 = moe.forward(c, dev["x"], dev["w_r"], dev["b"], ex, dev["shared"],
                                           want_routing=True,
                                           side_stream=None if one_stream else side)
    torch.cuda.synchronize()
    n_check = min(cfg.T, check_rows)
    check = dict(idx=idx2.cpu().numpy(), gate=gate2.cpu().numpy(), counts=counts2.cpu().numpy(),
                 out=o2[:n_check].double().cpu().numpy())
    del o2
    res = dict(cfg=cfg, elapsed=elapsed, ms_per_step=elapsed / steps * 1e3, stage_ms=avg,
               counts=counts_np, inputs=inp, step_spread=spread, step_ms=in_order, check=check,
               shared_expert=placement)
    if extra:
        res["next_rows"] = time_next_rows(moe, c, dev, counts, events, main)
    del dev, out
    torch.cuda.empty_cache()
    return res


# the V3-shaped prefill with the decode workload's fp8 e4m3 weights and
# 128 x 128 block scales
FP8_PREFILL = dict(w_dtype="fp8", w_block=128)


def fp8_prefill_summary(r):
    """Whole-forward rate and the routed up GEMM's MFMA rate (bf16 MFMAs on the
    dequantized weights) for the fp8-weight prefill."""
    cfg = r["cfg"]
    flops = 2.0 * up_rows(r) * cfg.d * 2 * cfg.inter
    up_ms = r["stage_ms"]["up"]
    return {"workload": "v3_prefill with fp8 e4m3 weights + 128x128 block scales",
            "shared_expert": r["shared_expert"],
            "ms_per_step": round(r["ms_per_step"], 4),
            "tokens_per_s": round(cfg.T / (r["ms_per_step"] * 1e-3), 1),
            "up_ms": round(up_ms, 4), "down_ms": round(r["stage_ms"]["down"], 4),
            "step_spread": r["step_spread"],
            "up_tflops": round(flops / (up_ms * 1e-3) / 1e12, 1),
            "up_frac_bf16_peak": round(flops / (up_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def up_rows(r):
    """Rows of the up-projection launch: the T*k routed slots, plus the T
    tokens of the shared expert when it is folded in as one more group."""
    cfg = r["cfg"]
    return cfg.T * cfg.k + (cfg.T if r["shared_expert"] == "folded" else 0)


def prefill_roofline(r):
    cfg = r["cfg"]
    flops = 2.0 * up_rows(r) * cfg.d * 2 * cfg.inter  # W1 and W3 over every row of the launch
    ms = r["stage_ms"]["up"]
    achieved = flops / (ms * 1e-3) / 1e12
    what = "routed + folded shared W1|W3" if r["shared_expert"] == "folded" else "routed W1|W3"
    return {"bound": "mfma", "kernel": f"gp::gemm_bf16_persist_kernel<32, 4, true, false> ({what} + SwiGLU)",
            "rows_per_launch": up_rows(r),
            "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "algorithmic_per_launch": flops, "avg_launch_ms": round(ms, 4),
            "traffic": traffic_from_profile("prefill_up" + ("_folded" if r["shared_expert"] == "folded" else ""),
                                            ["gemm_bf16_persist.hip", "grouped_sched.h"], flops)}


def decode_summary(r):
    cfg = r["cfg"]
    counts = r["counts"]
    n_active = int((counts > 0).sum())
    per_expert = cfg.expert_weight_bytes()  # fp8 W1, W3, W2 + fp32 block scales
    total_bytes = (n_active + cfg.n_shared) * per_expert
    ms = r["ms_per_step"]
    gbps = total_bytes / (ms * 1e-3) / 1e9
    # dominant kernel: the fp8 W1|W3 stream (2/3 of the active weight bytes) of the
    # active routed experts, and of the shared expert when it is folded in
    streamed = n_active + (cfg.n_shared if r["shared_expert"] == "folded" else 0)
    up_bytes = streamed * (2 * cfg.d * cfg.inter + 2 * (cfg.d // 128) * (cfg.inter // 128) * 4)
    up_ms = r["stage_ms"]["up"]
    up_gbps = up_bytes / (up_ms * 1e-3) / 1e9
    return {
        "workload": cfg.name, "T": cfg.T, "shared_expert": r["shared_expert"],
        "ms_per_step": round(ms, 4),
        "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "n_active_routed": n_active, "idle_experts": int(cfg.n_routed - n_active),
        "weight_bytes_per_step": total_bytes, "step_spread": r["step_spread"],
        "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
        "roofline": {"bound": "hbm", "kernel": "gemm_fp8_small_kernel<SwiGLU> (routed W1|W3 fp8)",
                     "achieved": round(up_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(up_gbps / PEAK_HBM_GBPS, 4), "algorithmic_per_launch": up_bytes,
                     "avg_launch_ms": round(up_ms, 4),
                     "traffic": traffic_from_profile(
                         "decode_up" + ("_folded" if r["shared_expert"] == "folded" else ""),
                         ["gemm_fp8.hip", "grouped_sched.h"], up_bytes)},
    }


TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}  # max |gpu - oracle| / RMS(oracle out)
TIE = 1e-6  # keys (or group scores) closer than this may select differently


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_leg(r, timed=False):
    """The fp64 oracle on the host cores: the benchmark's CPU leg, the only
    place it runs the oracle.  Routes all T tokens (near-tie count, agreement
    of the GPU's selected sets, per-expert counts and gates outside the tie
    window), then evaluates the layer output of the first rows the GPU run
    kept (its check forward) on the GPU's own selection (identical to the
    oracle's outside near ties) and compares them.  With ``timed`` the wall
    time of that output evaluation is the cpu_baseline (weight generation
    excluded: the experts the tokens use are drawn first)."""
    import numpy as np
    import oracle
    inp, cfg, chk = r["inputs"], r["cfg"], r["check"]
    N = cfg.n_routed
    x = inp.x()
    wr, b = inp.router_w(), inp.router_b()
    rt = oracle.route(cfg, oracle.widen(x, cfg.act_dtype), wr.astype(np.float64), b)
    near = rt["margin"] < TIE
    idx_g = chk["idx"].astype(np.int64)
    same = np.all(np.sort(idx_g, 1) == np.sort(rt["idx"], 1), axis=1)
    far = ~near
    counts_ok = bool(np.array_equal(np.bincount(idx_g[far].ravel(), minlength=N),
                                    np.bincount(rt["idx"][far].ravel(), minlength=N)))
    go = np.take_along_axis(rt["gates"], np.argsort(rt["idx"], 1), 1)[same]
    gg = np.take_along_axis(chk["gate"].astype(np.float64), np.argsort(idx_g, 1), 1)[same]
    gate_err = float((np.abs(go - gg) / np.maximum(np.abs(go), 1e-3)).max(initial=0.0))
    n = chk["out"].shape[0]
    sub = cfg.replace(T=n)
    xs = x[:n]
    needed = sorted(int(e) for e in np.unique(idx_g[:n]))
    st = inp.experts_stacked(experts=needed)
    cache = {e: {k: (None if v is None else v[j]) for k, v in st.items()} for j, e in enumerate(needed)}
    shared = inp.shared()
    t0 = time.perf_counter()
    res = oracle.forward(sub, xs, wr, b, lambda e: cache[e], shared, idx_override=idx_g[:n])
    dt = time.perf_counter() - t0
    ref, got = res["out"], chk["out"]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rms_d = float(np.sqrt(np.mean(res["delta"] ** 2)))
    err = float(np.abs(got - ref).max()) / rms
    err_d = float(np.abs(got - ref).max()) / rms_d
    import torch
    bf = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    mismatch = int((~same & far).sum())
    tol = TOL[cfg.w_dtype]
    parity = {"tokens_routed": int(cfg.T), "near_ties": int(near.sum()),
              "set_mismatch_outside_ties": mismatch, "counts_equal_outside_ties": counts_ok,
              "gate_max_rel_err": round(gate_err, 8), "output_tokens": int(n),
              "experts_in_output_check": len(needed),
              "err_rms_out": float(f"{err:.4e}"), "err_rms_delta": float(f"{err_d:.4e}"),
              "tol": tol, "bf16_output_floor": float(f"{float(np.abs(bf - ref).max()) / rms:.4e}"),
              "ok": bool(mismatch == 0 and counts_ok and gate_err < 2e-5 and err < tol)}
    base = None
    if timed:
        base = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": oracle_threads(),
                "kind": "oracle",
                "sample": f"first {n} tokens of {cfg.name} (T={cfg.T}): fp64 routing, "
                          f"{len(needed)} routed experts + shared MLP, {dt:.1f}s"}
    return base, parity


# the configurations besides the V3-shaped ones, timed and checked like them:
# GShard 16 x top-2 fp32 (aiany.app Step 2), DeepSeekMoE 1 + 63 top-7 (Step 6),
# the V2-shaped 2 + 160 top-6 (shivam2003.com "5.6", configuration table)
OTHER_CONFIGS = {"gshard_fp32": 512, "deepseekmoe_2b": 128, "v2_shaped": 32}  # rows checked
MALL_BYTES = 256 << 20
PEAK_FP32_TFLOPS = 157.3


def config_summary(r):
    cfg = r["cfg"]
    ms = r["ms_per_step"]
    flops = cfg.flops_per_token() * cfg.T
    tflops = flops / (ms * 1e-3) / 1e12
    wbytes = cfg.n_routed * cfg.expert_weight_bytes() + cfg.n_shared * cfg.expert_weight_bytes()
    out = {"T": cfg.T, "d": cfg.d, "n_routed": cfg.n_routed, "n_shared": cfg.n_shared,
           "inter": cfg.inter, "k": cfg.k, "dtype": cfg.w_dtype, "shared_expert": r["shared_expert"],
           "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "layer_tflops": round(tflops, 1),
           "layer_frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "step_spread": r["step_spread"],
           "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
           "weight_bytes": wbytes,
           "cache": ("weights fit the 256 MB Infinity Cache: resident across steps"
                     if wbytes < MALL_BYTES else "weights exceed the 256 MB Infinity Cache: read from HBM each step")}
    if cfg.w_dtype == "f32":
        out["layer_frac_fp32_peak"] = round(tflops / PEAK_FP32_TFLOPS, 4)
    return out


def summarize_trace(path, title=""):
    """Print a per-kernel table (calls, average and total duration, grouped by
    kernel and grid size) of a rocprofv3 kernel-trace CSV."""
    import collections
    import csv
    rows = list(csv.DictReader(open(path)))
    # launches of one kernel with one grid but on different streams (a
    # persistent grid serves the routed experts on the main stream and the
    # shared expert on the side stream) are listed apart: grid/stream
    agg = collections.defaultdict(list)
    for r in rows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = r.get("Grid_Size") or r.get("Grid_Size_X", "")
        agg[(r["Kernel_Name"], f"{grid}/s{r.get('Stream_Id', '?')}")].append(dur)
    total = sum(sum(v) for v in agg.values()) or 1
    if title:
        print(title)
    print(f"{'kernel':100s} {'grid/stream':>12s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name[:100]:100s} {grid:>12s} {len(v):6d} {sum(v) / len(v) / 1e3:10.2f} "
              f"{sum(v) / 1e6:10.3f} {100 * sum(v) / total:6.2f}")


def copy_calibration():
    """A plain elementwise copy of known size (reads and writes COPY_CAL_BYTES),
    launched three times so that the FETCH_SIZE / WRITE_SIZE counters of the
    same profiled process can be scaled to bytes."""
    import torch
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(fetch_csv, write_csv, command, folded=True):
    """Per-launch HBM traffic of the routed W1|W3 GEMMs from two rocprofv3
    --pmc runs of the same bench command (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the counter reads for the calibration copy.
    Writes the traffic summary under profiles/ and prints it."""
    import collections
    import csv

    def per_kernel(path, counter):
        # the routed and the shared launches of one kernel share its name and
        # (persistent) grid; the routed one moves several times more bytes, so
        # each kernel's figure is the mean over its dispatches above half its max
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            agg[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]) * 1024.0)
        out = {}
        for k, v in agg.items():
            big = [x for x in v if x >= 0.5 * max(v)]
            out[k] = sum(big) / len(big)
        return out

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(table, pred):
        keys = [k for k in table if pred(k[0])]
        return max(keys, key=lambda k: k[1]) if keys else None  # largest grid = routed launch

    cal_f = pick(fetch, lambda n: "MulFunctor" in n)
    cal_w = pick(write, lambda n: "MulFunctor" in n)
    sf = COPY_CAL_BYTES / fetch[cal_f]
    sw = COPY_CAL_BYTES / write[cal_w]
    db = read_traffic_db()  # entries of the other shared-expert placement are kept
    db["calibration"] = {"copy_bytes": COPY_CAL_BYTES, "fetch_counter_bytes": fetch[cal_f],
                         "write_counter_bytes": write[cal_w], "fetch_scale": sf, "write_scale": sw}
    suffix = "_folded" if folded else ""
    targets = {
        "prefill_up": (lambda n: "gemm_bf16_persist_kernel<32, 4, true, false>" in n,
                       ["gemm_bf16_persist.hip", "grouped_sched.h"]),
        "decode_up": (lambda n: "gemm_fp8_small_kernel<true" in n, ["gemm_fp8.hip", "grouped_sched.h"]),
    }
    for key, (pred, sources) in targets.items():
        kf, kw = pick(fetch, pred), pick(write, pred)
        if kf is None or kw is None:
            continue
        fb, wb = fetch[kf] * sf, write[kw] * sw
        db[key + suffix] = {"kernel": kf[0], "grid": kf[1], "fetch_bytes": round(fb),
                            "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb),
                            "shared_expert": "folded into the launch" if folded else "side stream",
                            "source_digest": source_digest(*sources)}
    header = ("# HBM traffic per launch of the routed W1|W3 GEMMs (rocprofv3 --pmc, two runs)\n"
              f"# command (run from /tmp, TMPDIR=/tmp), once with FETCH_SIZE and once with WRITE_SIZE:\n"
              f"#   {command}\n"
              "# each counter is scaled by its reading for a plain fp32 copy of "
              f"{COPY_CAL_BYTES >> 20} MiB read + {COPY_CAL_BYTES >> 20} MiB written\n"
              "# prefill_up = V3-shaped prefill (T=16384) routed up launch, decode_up = fp8 decode "
              "(T=64) routed up launch; *_folded = the same launches with the shared expert folded in as\n"
              "# one more group (bench.py's default), the others with it on a second stream (--two-streams);\n"
              "# source_digest pins the kernel sources\n")
    with open(TRAFFIC_FILE, "w") as f:
        f.write(header)
        f.write(json.dumps(db, indent=1) + "\n")
    print(header + json.dumps(db, indent=1))


def summarize_util(csv_path, command, out_path):
    """MFMA utilisation, clock and LDS bank conflicts per launch of the main
    GEMMs from one rocprofv3 --pmc run (GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE).
    rocprofv3 reports each counter summed over its hardware instances; the
    GPU-busy cycles GRBM_GUI_ACTIVE come from one instance per XCD."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names, dur = {}, {}
    for r in csv.DictReader(open(csv_path)):
        key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Dispatch_Id"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
        dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    n_xcd, simds = 8, 256 * 4
    targets = {"bf16 up (prefill)": "gemm_bf16_persist_kernel<32, 4, true, false>",
               "bf16 down (prefill)": "gemm_bf16_persist_kernel<32, 4, false, false>",
               # fp8 weights: any stage count (the second template argument)
               "fp8-weight up (prefill)": ", true, true>",
               "fp8-weight down (prefill)": ", false, true>",
               "fp8 up (decode)": "gemm_fp8_small_kernel<true, 4, 2>",
               "fp8 down (decode)": "gemm_fp8_small_kernel<false, 2, 3>"}
    lines = ["# MFMA utilisation of the main GEMM launches (rocprofv3 --pmc, one run)",
             "# command (run from /tmp, TMPDIR=/tmp):",
             f"#   {command}",
             "# summary: python bench.py --summarize-util <out>/bench_counter_collection.csv '<command>' <this file>",
             "# per kernel, its routed launches (largest grid, at least half the longest duration) averaged:",
             "#   cycles = GRBM_GUI_ACTIVE / 8 XCDs;",
             "#   clock = cycles / launch duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs);",
             "#   lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
             f"{'launch':34s} {'dispatches':>10s} {'ms':>8s} {'clock_GHz':>10s} {'mfma_busy':>10s} "
             f"{'lds_conflict':>13s}"]
    for label, pat in targets.items():
        keys = [k for k in per if pat in names[k]]
        if not keys:
            continue
        gmax = max(k[1] for k in keys)
        keys = [k for k in keys if k[1] == gmax]
        # the persistent grid is the same for the routed and the shared
        # launches; the routed ones run several times longer
        dmax = max(dur[k] for k in keys)
        keys = [k for k in keys if dur[k] >= 0.5 * dmax]
        n = len(keys)
        cyc = sum(per[k]["GRBM_GUI_ACTIVE"] for k in keys) / n / n_xcd
        ms = sum(dur[k] for k in keys) / n / 1e6
        mf = sum(per[k]["SQ_VALU_MFMA_BUSY_CYCLES"] for k in keys) / n
        lc = sum(per[k]["SQ_LDS_BANK_CONFLICT"] for k in keys)
        la = sum(per[k]["SQ_LDS_IDX_ACTIVE"] for k in keys)
        lines.append(f"{label:34s} {n:10d} {ms:8.3f} {cyc / (ms * 1e6):10.2f} {mf / (cyc * simds):10.3f} "
                     f"{(lc / la if la else 0.0):13.4f}")
    text = "\n".join(lines) + "\n"
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


def power_probe(out_path=None, reps=10):
    """The routed expert GEMMs of the V3-shaped prefill (moe_expert_ffn: up with
    SwiGLU, then down, on the workload's own routing) timed on the workload's
    activations and on all-zero activations of the same shape: the same
    instructions and memory traffic, different operand values.  Each case runs
    0.3 s back to back before `reps` event-timed calls."""
    import torch
    import datagen
    from datagen.device import upload
    import mixture_experts_ffn_gemm_amd as moe
    cfg = datagen.get_config("v3_prefill")
    dev = upload(datagen.MoEInputs(cfg))
    c = moe.config_from(cfg)
    idx, _ = moe.router(c, dev["x"], dev["w_r"], dev["b"])
    p = moe.permute(c, idx)
    ex = dev["experts"]
    rows = cfg.T * cfg.k
    x0 = torch.zeros_like(dev["x"])
    ws = moe.Workspace.get(c, "cuda")
    y = torch.empty((rows, cfg.d), dtype=dev["x"].dtype, device="cuda")
    events = HipEvents()
    rec = events.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    res = {}
    for name, xin in (("workload activations", dev["x"]), ("zero activations", x0),
                      ("workload activations again", dev["x"])):
        fn = lambda: moe.expert_ffn(c, cfg.n_routed, p["offsets"], rows, xin, ex["w1"], ex["w3"],
                                    ex["w2"], row_index=p["row_token"], y_rows=y, ws=ws)
        t_w = time.perf_counter()
        n = 0
        while time.perf_counter() - t_w < 0.3:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        e0, e1 = events.create(2)
        rec(e0, stream.cuda_stream)
        for _ in range(reps):
            fn()
        rec(e1, stream.cuda_stream)
        torch.cuda.synchronize()
        res[name] = events.elapsed_ms(e0, e1) / reps
        events.destroy([e0, e1])
    flops = 2.0 * rows * cfg.d * 3 * cfg.inter
    lines = ["# Routed expert GEMMs (up + SwiGLU, down) of the V3-shaped prefill, T=16384: operand-value",
             "# dependence of their speed (same launches, same memory traffic; the clock is set by power)",
             "# command: python bench.py --power-probe <this file>",
             f"{'activations':30s} {'ms (up + down)':>15s} {'TFLOP/s':>9s}"]
    for name, ms in res.items():
        lines.append(f"{name:30s} {ms:15.3f} {flops / (ms * 1e-3) / 1e12:9.1f}")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    print(text)


def padding_probe(out_path=None, reps=10):
    """The routed expert GEMMs of the V3-shaped prefill (moe_expert_ffn: up with
    SwiGLU, then down) on the workload's own routing, and on the same rows
    regrouped so that every expert owns exactly T*k/N = 512 of them (no
    partly filled 256-row tile): the same flops, gathers and weights, without
    the padding rows.  Each case runs 0.3 s back to back before `reps`
    event-timed calls."""
    import torch
    import datagen
    from datagen.device import upload
    import mixture_experts_ffn_gemm_amd as moe
    cfg = datagen.get_config("v3_prefill")
    dev = upload(datagen.MoEInputs(cfg), shared=False)
    c = moe.config_from(cfg)
    idx, _ = moe.router(c, dev["x"], dev["w_r"], dev["b"])
    p = moe.permute(c, idx)
    ex = dev["experts"]
    rows = cfg.T * cfg.k
    per = rows // cfg.n_routed
    uniform = torch.arange(0, rows + 1, per, dtype=torch.int32, device="cuda")
    counts = p["counts"].cpu().numpy()
    tiles_real = int(sum(-(-int(n) // 256) for n in counts))
    ws = moe.Workspace.get(c, "cuda")
    y = torch.empty((rows, cfg.d), dtype=dev["x"].dtype, device="cuda")
    events = HipEvents()
    rec = events.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    res = {}
    for name, off in (("workload routing", p["offsets"]), ("512 rows per expert", uniform),
                      ("workload routing again", p["offsets"])):
        fn = lambda: moe.expert_ffn(c, cfg.n_routed, off, rows, dev["x"], ex["w1"], ex["w3"],
                                    ex["w2"], row_index=p["row_token"], y_rows=y, ws=ws)
        t_w = time.perf_counter()
        n = 0
        while time.perf_counter() - t_w < 0.3:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        e0, e1 = events.create(2)
        rec(e0, stream.cuda_stream)
        for _ in range(reps):
            fn()
        rec(e1, stream.cuda_stream)
        torch.cuda.synchronize()
        res[name] = events.elapsed_ms(e0, e1) / reps
        events.destroy([e0, e1])
    flops = 2.0 * rows * cfg.d * 3 * cfg.inter
    lines = ["# Routed expert GEMMs (up + SwiGLU, down) of the V3-shaped prefill, T=16384: the cost of",
             "# partly filled 256-row tiles.  Same flops, gathered rows and weights; the second case",
             "# regroups the rows so every expert owns exactly 512 (no padding tile)",
             "# command: python bench.py --padding-probe <this file>",
             f"# M-tiles: workload routing {tiles_real} (counts min {counts.min()}, max {counts.max()}), "
             f"512 rows per expert {rows // 256}: {tiles_real / (rows // 256):.3f}x",
             f"{'rows per expert':30s} {'ms (up + down)':>15s} {'TFLOP/s':>9s}"]
    for name, ms in res.items():
        lines.append(f"{name:30s} {ms:15.3f} {flops / (ms * 1e-3) / 1e12:9.1f}")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    print(text)


STALL_A = ("GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
           "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM SQ_VALU_MFMA_BUSY_CYCLES")
STALL_B = ("GRBM_GUI_ACTIVE SQ_WAIT_INST_LDS SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
           "SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_MISC "
           "SQ_VALU_MFMA_COEXEC_CYCLES")


def summarize_stalls(csv_a, csv_b, command, out_path):
    """Where the wavefronts of the routed bf16 GEMMs spend their cycles, from two
    rocprofv3 --pmc passes (STALL_A, STALL_B) of the same command: every count
    as a fraction of the SIMD-cycles of the launch (GRBM_GUI_ACTIVE / 8 XCDs x
    1024 SIMDs; one wavefront per SIMD).  SQ_WAVE_CYCLES and the SQ_WAIT_*
    counters count in units of 4 cycles."""
    import collections
    import csv
    quad = {"SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"}
    targets = {"bf16 routed up": "gemm_bf16_persist_kernel<32, 4, true, false>",
               "bf16 routed down": "gemm_bf16_persist_kernel<32, 4, false, false>"}
    res = collections.defaultdict(dict)
    for path in (csv_a, csv_b):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
        for label, pat in targets.items():
            keys = [k for k in per if pat in names[k]]
            if not keys:
                continue
            gmax = max(per[k]["GRBM_GUI_ACTIVE"] for k in keys)
            keys = [k for k in keys if per[k]["GRBM_GUI_ACTIVE"] >= 0.5 * gmax]  # routed launches
            n = len(keys)
            simd_cycles = sum(per[k]["GRBM_GUI_ACTIVE"] for k in keys) / n / 8 * 1024
            for c in per[keys[0]]:
                if c == "GRBM_GUI_ACTIVE":
                    continue
                v = sum(per[k][c] for k in keys) / n * (4 if c in quad else 1)
                res[label][c] = (v / simd_cycles, n)
    lines = ["# Stall breakdown of the routed bf16 GEMM launches (rocprofv3 --pmc, two passes)",
             "# command of each pass (run from /tmp, TMPDIR=/tmp), counters STALL_A then STALL_B of bench.py:",
             f"#   {command}",
             "# summary: python bench.py --summarize-stalls <passA>/bench_counter_collection.csv "
             "<passB>/bench_counter_collection.csv '<command>' <this file>",
             "# fraction of the launch's SIMD-cycles (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), averaged over",
             "# the routed launches (at least half the longest); SQ_WAVE_CYCLES and SQ_WAIT_* count 4 cycles each",
             f"{'counter':30s} " + " ".join(f"{lab:>18s}" for lab in targets)]
    counters = sorted({c for lab in res for c in res[lab]})
    for c in counters:
        row = " ".join(f"{res[lab][c][0]:18.3f}" if c in res[lab] else f"{'-':>18s}" for lab in targets)
        lines.append(f"{c:30s} {row}")
    text = "\n".join(lines) + "\n"
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-util":
        summarize_util(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--power-probe":
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        power_probe(sys.argv[2] if len(sys.argv) > 2 else None)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--padding-probe":
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        padding_probe(sys.argv[2] if len(sys.argv) > 2 else None)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stalls":
        summarize_stalls(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else "")
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        # --summarize-pmc FETCH_CSV WRITE_CSV COMMAND [two-streams]
        summarize_pmc(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else "",
                      folded=not (len(sys.argv) > 5 and sys.argv[5] == "two-streams"))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager forwards instead of replays of one captured HIP graph")
    ap.add_argument("--no-fp8-prefill", action="store_true",
                    help="skip the V3-shaped prefill with fp8 block-scaled weights")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (the oracle: cpu_baseline and the parity records)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the GShard, DeepSeekMoE and V2-shaped configurations")
    ap.add_argument("--two-streams", action="store_true",
                    help="run the shared expert on a second stream instead of folding it into the "
                         "routed GEMMs (by default folded where it can be: bf16/fp8, one shared expert)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="launch a known-size copy first (scale for PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer is built and measured on a single "
              f"MI355X); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    events = HipEvents()
    if args.copy_calibration:
        copy_calibration()
    r = run_workload(args.workload, args.steps, args.warmup, events, extra=True,
                     two_streams=args.two_streams, graph=not args.no_graph)
    cfg = r["cfg"]
    value = cfg.T * args.steps / r["elapsed"]
    flops = cfg.flops_per_token() * cfg.T
    line = {
        "metric": "MoE-layer fwd tokens/s + MFMA % peak (V3 shape); decode HBM GB/s % peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.w_dtype, "data": "synthetic",
        "launch": "eager" if args.no_graph else "hip graph replay",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "n_routed": cfg.n_routed,
                   "n_shared": cfg.n_shared, "inter": cfg.inter, "k": cfg.k,
                   "groups": f"{cfg.topk_groups}/{cfg.n_groups}", "gate": cfg.gate,
                   "shared_expert": r["shared_expert"]},
        "layer_mfma_frac": round(flops / (r["ms_per_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_spread": r["step_spread"],
        "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
        "roofline": prefill_roofline(r),
        "next_rows": r.get("next_rows"),
    }
    legs = [(r, line, True)]  # (workload result, where its parity goes, timed cpu_baseline)
    if not args.no_fp8_prefill:
        f = run_workload("v3_prefill", max(2, args.steps // 2), args.warmup, events,
                         two_streams=args.two_streams, overrides=FP8_PREFILL,
                         graph=not args.no_graph, check_rows=8)
        line["next_rows"]["fp8_prefill"] = fp8_prefill_summary(f)
        legs.append((f, line["next_rows"]["fp8_prefill"], False))
    if not args.no_decode:
        d = run_workload("v3_decode", args.steps, args.warmup, events, two_streams=args.two_streams,
                         graph=not args.no_graph, check_rows=16)
        line["decode"] = decode_summary(d)
        legs.append((d, line["decode"], False))
    if not args.no_configs:
        line["configs"] = {}
        for name, rows in OTHER_CONFIGS.items():
            o = run_workload(name, args.steps, args.warmup, events, two_streams=args.two_streams,
                             graph=not args.no_graph, check_rows=rows)
            line["configs"][name] = config_summary(o)
            legs.append((o, line["configs"][name], False))
    if not args.no_cpu_baseline:
        for res, where, timed in legs:
            t0 = time.time()
            base, parity = cpu_leg(res, timed=timed)
            where["parity"] = parity
            if base is not None:
                line["cpu_baseline"] = base
            log(f"[bench] oracle leg {res['cfg'].name}{' (fp8 weights)' if res['cfg'].w_dtype == 'fp8' and res['cfg'].T > 64 else ''}: "
                f"{time.time() - t0:.1f}s, parity ok={parity['ok']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
