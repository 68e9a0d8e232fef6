"""Helpers shared by the GPU parity tests: oracle runs on seeded inputs and the
comparison rules (routing bit-exact outside near-ties, outputs relative to the
oracle output's RMS)."""
from __future__ import annotations

import sys

import numpy as np

import datagen
import oracle

TIE = 1e-6  # keys closer than this may legitimately select differently
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}


# one line per full-size comparison, printed at the end of the pytest run
# (tests/conftest.py), so that the figures show in the run's summary even
# when passing tests' output is captured
REPORT: list = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def report(line: str):
    REPORT.append(line)
    say(line)


def tol_for(cfg) -> float:
    return TOL[cfg.w_dtype]


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 1.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / max(rms, 1e-30)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def bf16_floor(ref: np.ndarray) -> float:
    """max |bf16(ref) - ref| / RMS(ref): the error a bf16 output has even when
    every value is the correctly rounded oracle value."""
    return rel_err(round_bf16(ref), ref)


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def oracle_route(cfg, inp: datagen.MoEInputs, x=None):
    x = inp.x() if x is None else x
    x64 = oracle.widen(x, cfg.act_dtype)
    return oracle.route(cfg, x64, inp.router_w().astype(np.float64), inp.router_b())


def check_routing(cfg, r, idx_gpu: np.ndarray, gate_gpu: np.ndarray, gate_tol=2e-5,
                  counts_gpu=None):
    """Selected sets equal the oracle's except for near-tie tokens, whose
    selection must still be a valid top-k within the tie window (keys within
    the window of the k-th, groups within the window of the last kept one, at
    most topk_groups groups).  Per-expert counts over the other tokens equal
    the oracle's; ``counts_gpu`` (the library's counts) must be the bincount of
    the GPU's selection.  Gates are compared per selected expert.  Returns
    (near_tie_count, order_diffs)."""
    T, k = idx_gpu.shape
    idx_o = r["idx"]
    near = r["margin"] < TIE
    N = cfg.n_routed
    if counts_gpu is not None:
        assert np.array_equal(np.asarray(counts_gpu), np.bincount(idx_gpu.ravel(), minlength=N))
    far = ~near
    assert np.array_equal(np.bincount(idx_gpu[far].ravel().astype(np.int64), minlength=N),
                          np.bincount(idx_o[far].ravel(), minlength=N)), \
        "per-expert counts over the tokens outside the tie window differ from the oracle's"
    so, sg = np.sort(idx_o, 1), np.sort(idx_gpu.astype(np.int64), 1)
    same = np.all(so == sg, axis=1)
    bad = ~same & ~near
    assert not bad.any(), (f"{int(bad.sum())} tokens select a different expert set outside the "
                           f"tie window; first {np.nonzero(bad)[0][:5]}: oracle {idx_o[bad][:2]} "
                           f"gpu {idx_gpu[bad][:2]} margins {r['margin'][bad][:2]}")
    # all selections are distinct, in range
    assert np.all((idx_gpu >= 0) & (idx_gpu < cfg.n_routed))
    assert np.all(np.diff(sg, axis=1) > 0)
    # near ties: every GPU pick must have a key within TIE of the k-th key and
    # lie in a group whose score is within TIE of the last kept group
    key = r.get("key_sel", r["key"])  # keys left after any expert exclusion
    mmargin = r.get("mmargin", np.full(T, np.inf))
    for t in np.nonzero(near & ~same)[0]:
        if mmargin[t] < TIE:  # the excluded set itself is inside the tie window
            continue
        kth = np.sort(key[t][r["allowed"][t]])[::-1][k - 1]
        assert np.all(key[t][idx_gpu[t]] >= kth - TIE), t
        if cfg.n_groups > 1:
            gsc = r["group_scores"][t]
            gs = cfg.n_routed // cfg.n_groups
            last = np.sort(gsc)[::-1][cfg.topk_groups - 1]
            assert np.all(gsc[idx_gpu[t] // gs] >= last - TIE), t
            assert len(np.unique(idx_gpu[t] // gs)) <= cfg.topk_groups, t
    # gates of the agreeing tokens, matched by expert id
    oi = np.argsort(idx_o, 1)
    gi = np.argsort(idx_gpu, 1)
    go = np.take_along_axis(r["gates"], oi, 1)[same]
    gg = np.take_along_axis(gate_gpu.astype(np.float64), gi, 1)[same]
    err = np.abs(go - gg) / np.maximum(np.abs(go), 1e-3)
    assert err.max(initial=0) < gate_tol, f"gate rel err {err.max()}"
    order_diff = int(np.sum(np.any(idx_o[same] != idx_gpu[same], axis=1)))
    return int(near.sum()), order_diff


def expert_cache(inp: datagen.MoEInputs, experts) -> dict:
    """The stored weights of the given routed experts, drawn on worker threads
    (the oracle then reads them one expert at a time)."""
    ids = sorted(set(int(e) for e in experts))
    if not ids:
        return {}
    st = inp.experts_stacked(experts=ids)
    return {e: {key: (None if v is None else v[j]) for key, v in st.items()}
            for j, e in enumerate(ids)}


def sample_tokens(idx: np.ndarray, n_routed: int, n_random: int, seed: int, tile: int = 256,
                  n_experts: int = 64) -> np.ndarray:
    """Tokens whose outputs are compared at full size: for n_experts experts
    spread over the expert range, the tokens of the first and last row of the
    expert's permuted rows and of the rows on either side of its first tile
    boundary (row offset + tile - 1, offset + tile), then n_random random
    tokens.  The permutation is the oracle's stable one of the GPU selection."""
    T = idx.shape[0]
    p = oracle.stable_permutation(idx.astype(np.int64), n_routed)
    off, row_token = p["offsets"], p["row_token"]
    picks = []
    for e in np.linspace(0, n_routed - 1, min(n_experts, n_routed)).round().astype(int):
        lo, hi = int(off[e]), int(off[e + 1])
        for r in (lo, hi - 1, lo + tile - 1, lo + tile):
            if lo <= r < hi:
                picks.append(int(row_token[r]))
    rng = np.random.default_rng(seed)
    picks.extend(rng.integers(0, T, n_random).tolist())
    return np.unique(np.array(picks, np.int64))
