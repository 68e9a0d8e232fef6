"""Plain fp64 CPU oracle of the DeepSeekMoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library: it widens the
stored inputs (bf16 / fp32 / e4m3 codes + block scales) to fp64 with its own
decoders and evaluates the layer's definition with numpy (BLAS dgemm for the
contractions), one expert at a time.

Sources (page title, then the section / equation followed):

* open-model-atlas, "DeepSeek-V3.2-Exp - Mixture of experts", "All 19 steps":
  router logits z = x W_r, sigmoid scores s = sigma(z), selection of the top-8
  of s+b inside the top-4 groups, gates G_i = 2.5 s_i / sum of the selected s;
  the routed expert g = x W1, u = x W3, a = g sigma(g), h = a (.) u, E = h W2;
  the same SwiGLU for the shared expert; Delta = sum_i G_i E_i + y_shared.
  Its parameter table and the excerpt of the reference forward (flatten the
  tokens, bincount the selections, skip experts with no token, accumulate the
  gate-weighted expert outputs in fp32, add the shared MLP) fix the data flow.
* aiany.app explainer of the DeepSeekMoE paper, Step 2: GShard routing is a
  dot product with every expert's centroid, a softmax over the routed scores,
  and the top-2 softmax values kept as the gates (no renormalisation).  Step 7:
  the routed and shared outputs are summed together with the layer input.
* shivam2003.com "5.6 The DeepSeekMoE Architecture", "Idea 2": output = sum of
  shared FFNs + sum of gated routed FFNs + x (residual).

Readings where the pages are silent (each is also listed in the design notes):

* group score = sum of the ``group_topn`` (=2) largest selection keys of the
  group; groups and experts tie-break towards the lower index;
* softmax mode: an optional per-expert offset b is added to the logits before
  the softmax (it moves both the selection and the gate values); gates are the
  unrenormalised selected probabilities times ``route_scale`` (1.0);
* sigmoid mode: b enters the selection key s+b only; the gate uses s;
* the residual x is added (``residual=False`` returns Delta alone);
* fp8 weights are e4m3fn codes times one fp32 scale per 128x128 block.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# decoders of the storage formats
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32 word."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_bits_to_f64(u8: np.ndarray) -> np.ndarray:
    """OCP e4m3fn bit patterns (uint8) -> float64, exactly.

    Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    u = np.asarray(u8, dtype=np.uint8).astype(np.int64)
    sign = np.where(u & 0x80, -1.0, 1.0)
    e = (u >> 3) & 0xF
    m = (u & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((u & 0x7) == 0x7), np.nan, v)


def dequant_fp8_blocks(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """codes [R, C] e4m3 x scales [R/block, C/block] fp32 -> fp64 [R, C]."""
    w = e4m3_bits_to_f64(codes)
    s = np.asarray(scales, dtype=np.float64)
    return w * np.repeat(np.repeat(s, block, axis=0), block, axis=1)


def widen(a, fmt: str, scales=None, block: int = 0) -> np.ndarray:
    """Stored tensor -> fp64.  fmt is 'f32', 'bf16' or 'fp8'."""
    if fmt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(a)
    if fmt == "fp8":
        return dequant_fp8_blocks(a, scales, block)
    raise ValueError(fmt)


def sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------


def router_logits(x64: np.ndarray, wr64: np.ndarray) -> np.ndarray:
    """z = x W_r.  x64 [T, d]; wr64 is W_r stored transposed, [N, d]."""
    return x64 @ wr64.T


def router_scores(gate: str, z: np.ndarray, b):
    """Returns (value, key): the per-expert score the gates use, and the key
    the selection ranks.

    softmax: p = softmax(z + b) over the routed experts only; key = p.
    sigmoid: s = sigma(z); key = s + b (b only steers the selection)."""
    if gate == "softmax":
        zz = z if b is None else z + np.asarray(b, np.float64)[None, :]
        e = np.exp(zz - zz.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        return p, p
    if gate == "sigmoid":
        s = sigmoid(z)
        key = s if b is None else s + np.asarray(b, np.float64)[None, :]
        return s, key
    raise ValueError(gate)


def _ranked(values: np.ndarray) -> np.ndarray:
    """Per row, column indices ordered by value descending, index ascending."""
    T, n = values.shape
    cols = np.broadcast_to(np.arange(n), (T, n))
    # lexsort: last key is primary
    return np.lexsort((cols, -values), axis=1)


def group_limit(key: np.ndarray, n_groups: int, topk_groups: int, group_topn: int):
    """Experts allowed by group-limited routing.

    The N experts form n_groups contiguous groups.  A group's score is the sum
    of its group_topn largest keys; the topk_groups best groups (lower group
    index on ties) stay eligible.  Returns (allowed [T,N] bool,
    group_scores [T,G], margin [T]) where margin is the gap between the last
    kept group's score and the best dropped one (inf if nothing is dropped)."""
    T, N = key.shape
    if n_groups <= 1:
        return np.ones((T, N), bool), key.sum(axis=1, keepdims=True), np.full(T, np.inf)
    gs = N // n_groups
    kg = key.reshape(T, n_groups, gs)
    top = -np.sort(-kg, axis=2)[:, :, :group_topn]
    gscore = top.sum(axis=2)
    order = _ranked(gscore)
    keep = order[:, :topk_groups]
    allowed_g = np.zeros((T, n_groups), bool)
    np.put_along_axis(allowed_g, keep, True, axis=1)
    allowed = np.repeat(allowed_g, gs, axis=1)
    if topk_groups < n_groups:
        last = np.take_along_axis(gscore, order[:, topk_groups - 1:topk_groups], 1)[:, 0]
        nxt = np.take_along_axis(gscore, order[:, topk_groups:topk_groups + 1], 1)[:, 0]
        margin = last - nxt
    else:
        margin = np.full(T, np.inf)
    return allowed, gscore, margin


def topk_select(key: np.ndarray, allowed: np.ndarray, k: int):
    """Top-k of the allowed keys, ordered key descending / index ascending.

    Returns (idx [T,k] int64, margin [T]) with margin = k-th minus (k+1)-th
    allowed key (inf if only k experts are allowed)."""
    masked = np.where(allowed, key, -np.inf)
    order = _ranked(masked)
    idx = order[:, :k]
    kth = np.take_along_axis(masked, order[:, k - 1:k], 1)[:, 0]
    if k < key.shape[1]:
        nxt = np.take_along_axis(masked, order[:, k:k + 1], 1)[:, 0]
        margin = np.where(np.isneginf(nxt), np.inf, kth - nxt)
    else:
        margin = np.full(key.shape[0], np.inf)
    return idx, margin


def gate_values(gate: str, route_scale: float, value: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """softmax: G = route_scale * p_sel (unrenormalised).
    sigmoid: G = route_scale * s_sel / sum(s_sel)."""
    sel = np.take_along_axis(value, idx, axis=1)
    if gate == "softmax":
        return route_scale * sel
    return route_scale * sel / sel.sum(axis=1, keepdims=True)


def exclude_experts(key: np.ndarray, allow=None, mask_top: int = 0):
    """Keys with experts taken out of the selection.

    aiany.app explainer, Step 9, probe 1: for each token the routed experts the
    router wanted most are masked and the token routes among the rest.  Here
    ``allow`` (bool [N], optional) first removes a fixed expert set, then each
    token's ``mask_top`` highest remaining keys (key descending, index
    ascending, as in the top-k) are removed.  Removed keys become -inf; the
    scores themselves (softmax probabilities, sigmoid values) are unchanged.
    Returns (keys, margin) with margin = the mask_top-th minus the next
    remaining key (inf when nothing is masked per token)."""
    masked = np.array(key, dtype=np.float64, copy=True)
    if allow is not None:
        masked[:, ~np.asarray(allow, bool)] = -np.inf
    margin = np.full(masked.shape[0], np.inf)
    if mask_top > 0:
        order = _ranked(masked)
        last = np.take_along_axis(masked, order[:, mask_top - 1:mask_top], 1)[:, 0]
        nxt = np.take_along_axis(masked, order[:, mask_top:mask_top + 1], 1)[:, 0]
        margin = last - nxt
        np.put_along_axis(masked, order[:, :mask_top], -np.inf, axis=1)
    return masked, margin


def route(cfg, x64: np.ndarray, wr64: np.ndarray, b=None, allow=None, mask_top: int = 0) -> dict:
    """Router of the layer for every token of x64.  cfg needs k, n_groups,
    topk_groups, group_topn, gate, route_scale, n_routed.  ``allow`` and
    ``mask_top`` take experts out of the selection (``exclude_experts``)."""
    z = router_logits(x64, wr64)
    value, key = router_scores(cfg.gate, z, b)
    key_sel, mmargin = exclude_experts(key, allow, mask_top)
    allowed, gscore, gmargin = group_limit(key_sel, cfg.n_groups, cfg.topk_groups,
                                           cfg.group_topn)
    idx, kmargin = topk_select(key_sel, allowed, cfg.k)
    gates = gate_values(cfg.gate, cfg.route_scale, value, idx)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_routed)
    return dict(z=z, value=value, key=key, key_sel=key_sel, allowed=allowed,
                group_scores=gscore, idx=idx, gates=gates, counts=counts,
                margin=np.minimum(np.minimum(kmargin, gmargin), mmargin),
                kmargin=kmargin, gmargin=gmargin, mmargin=mmargin)


def bias_update(b, counts, slots: int, gamma: float) -> np.ndarray:
    """Auxiliary-loss-free balancing step.

    grasp.study lesson, 3.2 "Auxiliary-Loss-Free Load Balancing": after a batch,
    each expert's selection bias moves by a fixed step, up when the expert was
    underloaded and down when it was overloaded (shivam2003.com "5.6", the
    V3 column of the configuration table: balancing by that bias instead of
    auxiliary losses).  Reading: the load of expert i is its count of the
    ``slots`` = T*k selections, the reference is the mean slots/N, the step is
    gamma * sign(mean - load_i) (no change at exactly the mean); the sign is
    decided on integers (N*load_i against slots); b is the fp32 router bias, so
    the updated value is rounded to fp32 once."""
    counts = np.asarray(counts, np.int64)
    n = counts.size
    sgn = np.sign(np.int64(slots) - counts * n).astype(np.float64)
    return (np.asarray(b, np.float32).astype(np.float64) +
            np.float64(np.float32(gamma)) * sgn).astype(np.float32)


def stable_permutation(idx: np.ndarray, n_routed: int) -> dict:
    """Expert-major order of the T*k slots (slot f = t*k + j), stable in f.

    Returns counts [N], offsets [N+1], row_token [T*k] (token of each permuted
    row) and slot_row [T*k] (permuted row of each slot)."""
    T, k = idx.shape
    flat = idx.reshape(-1)
    perm = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=n_routed)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_row = np.empty_like(perm)
    slot_row[perm] = np.arange(perm.size)
    return dict(counts=counts, offsets=offsets, row_token=perm // k, slot_row=slot_row,
                perm=perm)


# ----------------------------------------------------------------------------
# experts and the layer
# ----------------------------------------------------------------------------


def swiglu(x64: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """E(x) = (silu(x W1) (.) x W3) W2 with silu(g) = g sigma(g).

    w1, w3 are W1, W3 stored transposed ([I, d]); w2 is W2 transposed ([d, I])."""
    g = x64 @ w1.T
    u = x64 @ w3.T
    h = g * sigmoid(g) * u
    return h @ w2.T


def expert_weights64(cfg, ex: dict):
    """Widen one expert's stored weights (dict w1, w3, w2 [+ s1, s3, s2])."""
    fmt, blk = cfg.w_dtype, cfg.w_block
    return (widen(ex["w1"], fmt, ex.get("s1"), blk),
            widen(ex["w3"], fmt, ex.get("s3"), blk),
            widen(ex["w2"], fmt, ex.get("s2"), blk))


def combine_outputs(x64, idx, gates, get_expert, shared, cfg, residual=True,
                    tokens=None) -> dict:
    """Delta = sum_j G_j E_{idx_j}(x) + y_shared, and out = x + Delta.

    Evaluates only the experts selected by the tokens considered (experts with
    no token are never touched), one expert at a time.  ``tokens`` selects a
    subset of rows of x64/idx/gates (default: all)."""
    if tokens is not None:
        x64, idx, gates = x64[tokens], idx[tokens], gates[tokens]
    T = x64.shape[0]
    y_routed = np.zeros_like(x64)
    for e in np.unique(idx):
        rows, cols = np.nonzero(idx == e)
        w1, w3, w2 = expert_weights64(cfg, get_expert(int(e)))
        y_routed[rows] += gates[rows, cols][:, None] * swiglu(x64[rows], w1, w3, w2)
    y_shared = np.zeros_like(x64)
    if shared is not None:
        w1, w3, w2 = expert_weights64(cfg, shared)
        y_shared = swiglu(x64, w1, w3, w2)
    delta = y_routed + y_shared
    out = x64 + delta if residual else delta
    return dict(y_routed=y_routed, y_shared=y_shared, delta=delta, out=out, T=T)


def forward(cfg, x_stored, wr, b, get_expert, shared, tokens=None, residual=True,
            idx_override=None) -> dict:
    """The whole layer: route every token, then evaluate the outputs of
    ``tokens`` (default all).  ``idx_override`` [T,k] replaces the selection
    (its gates are recomputed from the same scores) - used to evaluate a
    selection that differs from the oracle's only inside a near-tie."""
    x64 = widen(x_stored, cfg.act_dtype)
    wr64 = np.asarray(wr, np.float32).astype(np.float64)
    r = route(cfg, x64, wr64, b)
    idx = r["idx"] if idx_override is None else np.asarray(idx_override, np.int64)
    gates = r["gates"] if idx_override is None else gate_values(
        cfg.gate, cfg.route_scale, r["value"], idx)
    res = combine_outputs(x64, idx, gates, get_expert, shared, cfg, residual, tokens)
    res.update(route=r, idx=idx, gates=gates, x64=x64 if tokens is None else x64[tokens])
    return res
