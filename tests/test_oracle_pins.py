"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself: values
printed on the pages (tests/golden/), hand-worked examples, closed forms,
library routines (torch CPU) and brute force over every subset on tiny
inputs.  A plausible slip in the oracle (a dropped residual, a renormalised
softmax gate, the bias leaking into sigmoid gates, a missing group limit, a
wrong group score, W1/W3 swapped, a transposed operand, an unstable
permutation) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


class Cfg:
    """A minimal router/expert configuration for hand-made cases."""

    def __init__(self, **kw):
        self.k = 2
        self.n_groups = 1
        self.topk_groups = 1
        self.group_topn = 2
        self.gate = "softmax"
        self.route_scale = 1.0
        self.n_routed = 4
        self.act_dtype = "f32"
        self.w_dtype = "f32"
        self.w_block = 0
        self.__dict__.update(kw)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoders


def test_bf16_decoder_matches_torch_on_every_code():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x38] == 1.0


def test_fp8_block_dequant_hand_values():
    # four 128x128 blocks with distinct scales; code 0x38 is 1.0, 0x40 is 2.0
    codes = np.full((256, 256), 0x38, np.uint8)
    codes[200, 3] = 0x40
    scales = np.array([[0.5, 2.0], [3.0, 0.25]], np.float32)
    w = oracle.dequant_fp8_blocks(codes, scales, 128)
    assert w[0, 0] == 0.5 and w[0, 255] == 2.0 and w[255, 0] == 3.0 and w[255, 255] == 0.25
    assert w[200, 3] == 6.0  # block (1,0): 2.0 * 3.0


def test_datagen_fp8_roundtrip_within_half_ulp():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((256, 384)).astype(np.float32) * 0.02
    q, s = datagen.quantize_fp8_blocks(w)
    back = oracle.dequant_fp8_blocks(q, s, 128)
    # e4m3 has 3 mantissa bits: relative spacing 2^-3, half-ulp 2^-4 (normals)
    blk_amax = np.repeat(np.repeat(np.abs(w).reshape(2, 128, 3, 128).max(axis=(1, 3)), 128, 0), 128, 1)
    err = np.abs(back - w)
    assert np.all(err <= np.maximum(np.abs(w) * 2.0 ** -4, blk_amax / 448 * 2.0 ** -10) + 1e-12)


# ---------------------------------------------------------------- pages' numbers


def test_v3_parameter_accounting_from_generated_shapes(golden_dir):
    g = _golden(golden_dir, "pages_numbers.json")["v3_block_parameters"]
    cfg = datagen.get_config("v3_prefill")
    inp = datagen.MoEInputs(cfg)
    wr, b = inp.router_w(), inp.router_b()
    router = wr.size + b.size
    ex = inp.expert(0)
    expert = ex["w1"].size + ex["w3"].size + ex["w2"].size
    sh = inp.shared()
    shared = sh["w1"].size + sh["w3"].size + sh["w2"].size
    assert router == g["router"]
    assert expert == g["routed_expert"]
    assert cfg.n_routed * expert == g["routed_total"]
    assert shared == g["shared_expert"]
    assert router + cfg.n_routed * expert + shared == g["per_block"]
    assert g["per_block"] * g["moe_blocks"] == g["all_blocks"]
    # the decode workload stores the same count of weights (fp8 codes)
    dec = datagen.MoEInputs(datagen.get_config("v3_decode")).expert(7)
    assert dec["w1"].size + dec["w3"].size + dec["w2"].size == g["routed_expert"]
    assert dec["s1"].shape == (2048 // 128, 7168 // 128) and dec["s2"].shape == (7168 // 128, 2048 // 128)


def _enumerate_topk_outcomes(n, k):
    """Drive the oracle's top-k with an indicator-like key for every k-subset
    and collect the distinct selections it returns."""
    outcomes = set()
    base = np.arange(n, dtype=np.float64) * 1e-3  # distinct background keys
    for sub in itertools.combinations(range(n), k):
        key = base.copy()
        key[list(sub)] += 1.0
        idx, _ = oracle.topk_select(key[None, :], np.ones((1, n), bool), k)
        got = tuple(sorted(idx[0].tolist()))
        assert got == sub
        outcomes.add(got)
    return len(outcomes)


def test_combinations_by_enumeration(golden_dir):
    g = _golden(golden_dir, "pages_numbers.json")["combinations"]
    assert _enumerate_topk_outcomes(16, 2) == g["c16_2"]["value"]
    assert _enumerate_topk_outcomes(8, 2) == g["c8_2"]["value"]


def test_combinations_closed_form(golden_dir):
    g = _golden(golden_dir, "pages_numbers.json")["combinations"]
    assert math.comb(64, 8) == g["c64_8"]["value"]
    assert math.comb(63, 7) == g["c63_7"]["value"]
    assert round(math.comb(64, 8) / math.comb(16, 2) / 1e6) == g["fold_16_2_to_64_8_millions"]["value"]
    n = math.comb(64, 16)
    assert 0.99 * g["nearly_489_trillion"]["value"] < n < g["nearly_489_trillion"]["value"]
    # fine-grained segmentation keeps the active width: m*k*(d_ff/m) = k*d_ff
    for m in (1, 2, 4, 8):
        assert (m * 2) * (2048 // m) == 2 * 2048


# ---------------------------------------------------------------- top-k


def test_topk_brute_force_ungrouped():
    rng = np.random.default_rng(1)
    for trial in range(200):
        n = int(rng.integers(2, 13))
        k = int(rng.integers(1, n + 1))
        key = rng.standard_normal(n)
        idx, margin = oracle.topk_select(key[None, :], np.ones((1, n), bool), k)
        best = max(itertools.combinations(range(n), k), key=lambda s: key[list(s)].sum())
        assert set(idx[0].tolist()) == set(best)
        assert np.all(np.diff(key[idx[0]]) < 0)  # ordered by key descending
        rest = sorted(set(range(n)) - set(best), key=lambda i: -key[i])
        if rest:
            assert np.isclose(margin[0], key[idx[0, -1]] - key[rest[0]])


def _brute_grouped(key, n_groups, topk_groups, topn, k):
    n = key.size
    gs = n // n_groups
    groups = [list(range(g * gs, (g + 1) * gs)) for g in range(n_groups)]
    gscore = [max(sum(key[list(c)]) for c in itertools.combinations(grp, topn)) for grp in groups]
    best_groups = max(itertools.combinations(range(n_groups), topk_groups),
                      key=lambda s: sum(gscore[i] for i in s))
    allowed = [e for g in best_groups for e in groups[g]]
    return set(max(itertools.combinations(allowed, k), key=lambda s: key[list(s)].sum()))


def test_topk_brute_force_grouped():
    rng = np.random.default_rng(2)
    for trial in range(150):
        n_groups = int(rng.choice([2, 3, 4]))
        gs = int(rng.integers(2, 4))
        n = n_groups * gs
        topk_groups = int(rng.integers(1, n_groups + 1))
        k = int(rng.integers(1, topk_groups * gs + 1))
        key = rng.standard_normal(n)
        allowed, gscore, gmargin = oracle.group_limit(key[None, :], n_groups, topk_groups, 2)
        idx, _ = oracle.topk_select(key[None, :], allowed, k)
        assert set(idx[0].tolist()) == _brute_grouped(key, n_groups, topk_groups, 2, k)
        # group scores and the margin by brute force: the best pair sum of each
        # group, sorted; the margin is the last kept score minus the best dropped
        bs = sorted((max(key[a] + key[b] for a, b in itertools.combinations(range(g * gs, (g + 1) * gs), 2))
                     for g in range(n_groups)), reverse=True)
        assert np.allclose(np.sort(gscore[0])[::-1], bs, rtol=0, atol=1e-15)
        if topk_groups < n_groups:
            assert np.isclose(gmargin[0], bs[topk_groups - 1] - bs[topk_groups], rtol=0, atol=1e-15)
        else:
            assert np.isinf(gmargin[0])


def test_softmax_logit_offset_hand_example(golden_dir):
    """Softmax routing with a per-expert logit offset, worked by hand: the
    offset moves both the selection and the gate values, the gates are the
    unrenormalised probabilities, equal keys go to the lower index."""
    g = _golden(golden_dir, "softmax_offset_example.json")
    x = np.array(g["x"], np.float32)
    wr = np.array(g["w_r"], np.float32)
    b = np.array(g["b"], np.float32)
    tol = g["tolerance"]
    cfg = Cfg(n_routed=g["n_routed"], k=g["k"], gate="softmax", route_scale=g["route_scale"])
    r = oracle.route(cfg, x.astype(np.float64), wr.astype(np.float64), b)
    assert np.array_equal(r["z"][0] + b.astype(np.float64), np.array(g["logits_plus_offset"]))
    assert np.allclose(r["value"][0], g["expected_p"], rtol=0, atol=tol)
    assert r["idx"][0].tolist() == g["expected_idx"]
    assert np.allclose(r["gates"][0], g["expected_gates"], rtol=0, atol=tol)
    r3 = oracle.route(Cfg(n_routed=g["n_routed"], k=3, gate="softmax"), x.astype(np.float64),
                      wr.astype(np.float64), b)
    assert r3["idx"][0].tolist() == g["k3_expected_idx"]
    assert np.allclose(r3["gates"][0], g["k3_expected_gates"], rtol=0, atol=tol)


def test_softmax_offset_shift_invariance():
    """A softmax is unchanged when every logit moves by the same amount: an
    offset that is constant over the experts selects and gates exactly as no
    offset, and adding a constant to a non-constant offset changes nothing;
    the same non-constant offset does change the probabilities."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((200, 16))
    wr = rng.standard_normal((10, 16)) / 4
    cfg = Cfg(n_routed=10, k=3, gate="softmax")
    base = oracle.route(cfg, x, wr)
    const = oracle.route(cfg, x, wr, np.full(10, 0.75, np.float32))
    assert np.array_equal(base["idx"], const["idx"])
    assert np.allclose(base["gates"], const["gates"], rtol=1e-13, atol=0)
    off = rng.normal(0, 0.5, 10).astype(np.float32)
    a = oracle.route(cfg, x, wr, off)
    shifted = oracle.route(cfg, x, wr, (off + np.float32(2.0)).astype(np.float32))
    assert np.array_equal(a["idx"], shifted["idx"])
    assert np.allclose(a["gates"], shifted["gates"], rtol=1e-6, atol=0)
    # probabilities of softmax(z + b) by torch, as a second definition
    p = torch.softmax(torch.from_numpy(x @ wr.T + off.astype(np.float64)), dim=1).numpy()
    assert np.allclose(a["value"], p, rtol=1e-12, atol=0)
    assert not np.allclose(a["value"], base["value"])


def test_grouped_hand_example(golden_dir):
    g = _golden(golden_dir, "grouped_routing_example.json")
    cfg = Cfg(n_routed=g["n_routed"], n_groups=g["n_groups"], topk_groups=g["topk_groups"],
              group_topn=g["group_topn"], k=g["k"], gate="sigmoid", route_scale=g["route_scale"])
    x = np.ones((1, 4))
    wr = np.zeros((g["n_routed"], 4))  # z = 0 -> s = 0.5 exactly
    r = oracle.route(cfg, x, wr, np.array(g["b"]))
    assert np.array_equal(r["key"][0], np.array(g["keys"]))
    assert np.array_equal(r["group_scores"][0], np.array(g["group_scores"]))
    assert r["idx"][0].tolist() == g["expected_idx"]
    assert np.allclose(r["gates"][0], g["expected_gates"], rtol=0, atol=1e-15)
    r2 = oracle.route(cfg, x, wr, np.array(g["case2_b"]))
    assert r2["idx"][0].tolist() == g["case2_expected_idx"]


def test_zero_router_tie_break_and_gates():
    # softmax: uniform p = 1/N, experts 0..k-1, gates 1/N
    x = np.random.default_rng(3).standard_normal((5, 8))
    cfg = Cfg(n_routed=16, k=2, gate="softmax")
    r = oracle.route(cfg, x, np.zeros((16, 8)))
    assert np.array_equal(r["idx"], np.tile([0, 1], (5, 1)))
    assert np.allclose(r["gates"], 1 / 16, rtol=0, atol=1e-16)
    # V3 shape: groups 0..3 kept, experts 0..7 selected, gates 2.5/8
    cfg = Cfg(n_routed=256, k=8, n_groups=8, topk_groups=4, gate="sigmoid", route_scale=2.5)
    r = oracle.route(cfg, x, np.zeros((256, 8)), np.zeros(256))
    assert np.array_equal(r["idx"], np.tile(np.arange(8), (5, 1)))
    assert np.all(r["allowed"][:, :128]) and not np.any(r["allowed"][:, 128:])
    assert np.allclose(r["gates"], 2.5 / 8, rtol=0, atol=1e-15)


def test_gate_definitions_on_random_inputs():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 32))
    wr = rng.standard_normal((256, 32)) / np.sqrt(32)
    b = rng.uniform(-0.05, 0.05, 256)
    cfg = Cfg(n_routed=256, k=8, n_groups=8, topk_groups=4, gate="sigmoid", route_scale=2.5)
    r = oracle.route(cfg, x, wr, b)
    assert np.allclose(r["gates"].sum(axis=1), 2.5, rtol=0, atol=4e-15)
    s = 1 / (1 + np.exp(-(x @ wr.T)))
    assert np.allclose(r["gates"], 2.5 * np.take_along_axis(s, r["idx"], 1)
                       / np.take_along_axis(s, r["idx"], 1).sum(1, keepdims=True))
    # every selected expert lies in an allowed group; there are exactly 4 of them
    assert np.all(np.take_along_axis(r["allowed"], r["idx"], 1))
    assert np.all(r["allowed"].reshape(64, 8, 32).all(2).sum(1) == 4)
    cfg = Cfg(n_routed=63, k=7, gate="softmax")
    wr = rng.standard_normal((63, 32)) / np.sqrt(32)
    r = oracle.route(cfg, x, wr)
    p = torch.softmax(torch.from_numpy(x @ wr.T), dim=1).numpy()
    assert np.allclose(r["value"], p, rtol=1e-13, atol=0)
    assert np.allclose(r["value"].sum(1), 1.0)
    assert np.all(r["gates"].sum(1) < 1.0)
    assert np.allclose(r["gates"], np.take_along_axis(p, r["idx"], 1), rtol=1e-13)


# ---------------------------------------------------------------- experts / layer


def _torch_swiglu(x, w1, w3, w2):
    """Textbook SwiGLU MLP via torch (CPU fp64): (silu(x W1) * x W3) W2."""
    X = torch.from_numpy(x)
    return ((torch.nn.functional.silu(X @ torch.from_numpy(w1).T) * (X @ torch.from_numpy(w3).T))
            @ torch.from_numpy(w2).T).numpy()


def _rand_experts(rng, n, d, I):
    return [dict(w1=(rng.standard_normal((I, d)) / np.sqrt(d)).astype(np.float32),
                 w3=(rng.standard_normal((I, d)) / np.sqrt(d)).astype(np.float32),
                 w2=(rng.standard_normal((d, I)) / np.sqrt(I)).astype(np.float32)) for _ in range(n)]


def test_closed_form_two_of_four_softmax_layer():
    """d=2, N=4, I=1: every quantity has a closed form."""
    x = np.array([[1.0, 0.0]], np.float32)
    wr = np.array([[2.0, 0.0], [1.0, 0.0], [0.0, 5.0], [0.0, -5.0]], np.float32)  # z = 2,1,0,0
    experts = [
        dict(w1=np.array([[1.0, 0]], np.float32), w3=np.array([[2.0, 0]], np.float32),
             w2=np.array([[1.0], [-1.0]], np.float32)),
        dict(w1=np.array([[-1.0, 0]], np.float32), w3=np.array([[1.0, 0]], np.float32),
             w2=np.array([[0.5], [2.0]], np.float32)),
        dict(w1=np.array([[9.0, 0]], np.float32), w3=np.array([[9.0, 0]], np.float32),
             w2=np.array([[9.0], [9.0]], np.float32)),
        dict(w1=np.array([[9.0, 0]], np.float32), w3=np.array([[9.0, 0]], np.float32),
             w2=np.array([[9.0], [9.0]], np.float32)),
    ]
    cfg = Cfg(n_routed=4, k=2, gate="softmax")
    res = oracle.forward(cfg, x, wr, None, lambda e: experts[e], None)
    Z = math.exp(2) + math.exp(1) + 2.0
    p0, p1 = math.exp(2) / Z, math.exp(1) / Z
    sig = lambda v: 1 / (1 + math.exp(-v))
    e0 = 1.0 * sig(1.0) * 2.0                    # h for expert 0
    e1 = -1.0 * sig(-1.0) * 1.0                  # h for expert 1
    want = np.array([1.0 + p0 * e0 * 1.0 + p1 * e1 * 0.5,
                     0.0 + p0 * e0 * -1.0 + p1 * e1 * 2.0])
    assert res["idx"][0].tolist() == [0, 1]
    assert np.allclose(res["gates"][0], [p0, p1], rtol=1e-15)
    assert np.allclose(res["out"][0], want, rtol=1e-14, atol=1e-15)
    delta = oracle.forward(cfg, x, wr, None, lambda e: experts[e], None, residual=False)["out"]
    assert np.allclose(delta[0], want - np.array([1.0, 0.0]), rtol=1e-14, atol=1e-15)


def test_single_expert_reduces_to_dense_swiglu():
    rng = np.random.default_rng(5)
    d, I, T = 24, 40, 17
    x = rng.standard_normal((T, d)).astype(np.float32)
    ex = _rand_experts(rng, 1, d, I)
    cfg = Cfg(n_routed=1, k=1, gate="softmax")
    res = oracle.forward(cfg, x, rng.standard_normal((1, d)).astype(np.float32), None,
                         lambda e: ex[e], None)
    x64 = x.astype(np.float64)
    want = x64 + _torch_swiglu(x64, *(ex[0][k].astype(np.float64) for k in ("w1", "w3", "w2")))
    assert np.allclose(res["gates"], 1.0)
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_dispatch_equals_dense_masked_sum(gate):
    """sum over ALL experts of G_i E_i (G_i = 0 when unselected), every expert
    evaluated on every token with torch, equals the oracle's dispatch form."""
    rng = np.random.default_rng(6)
    T, d, I, N, S = 40, 16, 24, 12, 2
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((N, d)) / 4).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    ex = _rand_experts(rng, N, d, I)
    shared_parts = _rand_experts(rng, S, d, I)
    shared = dict(w1=np.concatenate([s["w1"] for s in shared_parts]),
                  w3=np.concatenate([s["w3"] for s in shared_parts]),
                  w2=np.concatenate([s["w2"] for s in shared_parts], axis=1))
    kw = dict(n_groups=4, topk_groups=2, gate="sigmoid", route_scale=2.5) if gate == "sigmoid" else {}
    cfg = Cfg(n_routed=N, k=3, **kw)
    res = oracle.forward(cfg, x, wr, b, lambda e: ex[e], shared)
    x64 = x.astype(np.float64)
    dense_g = np.zeros((T, N))
    np.put_along_axis(dense_g, res["idx"], res["gates"], axis=1)
    want = x64.copy()
    for e in range(N):
        want += dense_g[:, e:e + 1] * _torch_swiglu(x64, *(ex[e][k].astype(np.float64) for k in ("w1", "w3", "w2")))
    for s in shared_parts:  # S experts of width I == one MLP of width S*I
        want += _torch_swiglu(x64, *(s[k].astype(np.float64) for k in ("w1", "w3", "w2")))
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)


def test_all_experts_on_equals_probability_weighted_sum():
    rng = np.random.default_rng(7)
    T, d, I, N = 9, 8, 12, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((N, d)).astype(np.float32)
    ex = _rand_experts(rng, N, d, I)
    cfg = Cfg(n_routed=N, k=N, gate="softmax")
    res = oracle.forward(cfg, x, wr, None, lambda e: ex[e], None)
    x64 = x.astype(np.float64)
    p = torch.softmax(torch.from_numpy(x64 @ wr.astype(np.float64).T), 1).numpy()
    want = x64 + sum(p[:, e:e + 1] * _torch_swiglu(x64, *(ex[e][k].astype(np.float64) for k in ("w1", "w3", "w2")))
                     for e in range(N))
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)


def test_segmentation_identity():
    """An expert cut into m column slices of its intermediate width, outputs
    summed, equals the whole expert (fine-grained segmentation's ledger)."""
    rng = np.random.default_rng(8)
    d, I, m = 16, 32, 4
    x = rng.standard_normal((7, d))
    w1, w3 = rng.standard_normal((I, d)), rng.standard_normal((I, d))
    w2 = rng.standard_normal((d, I))
    whole = oracle.swiglu(x, w1, w3, w2)
    sl = I // m
    parts = sum(oracle.swiglu(x, w1[i * sl:(i + 1) * sl], w3[i * sl:(i + 1) * sl], w2[:, i * sl:(i + 1) * sl])
                for i in range(m))
    assert np.allclose(whole, parts, rtol=1e-12, atol=1e-12)
    # and it is not symmetric in W1 / W3 (silu acts on x W1 only)
    assert not np.allclose(whole, oracle.swiglu(x, w3, w1, w2))


def test_stable_permutation_brute_force():
    rng = np.random.default_rng(9)
    T, k, N = 50, 3, 7
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)])
    p = oracle.stable_permutation(idx, N)
    assert np.array_equal(p["counts"], [int((idx == e).sum()) for e in range(N)])
    row = 0
    for e in range(N):
        assert p["offsets"][e] == row
        for t in range(T):  # tokens ascending within an expert
            for j in range(k):
                if idx[t, j] == e:
                    assert p["row_token"][row] == t
                    assert p["slot_row"][t * k + j] == row
                    row += 1
    assert row == T * k == p["offsets"][N]


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_idx_override_recomputes_gates(gate):
    """forward(idx_override=...) with a selection other than the oracle's own:
    the gates are those of the overriding experts, recomputed from the same
    scores (aiany.app Step 2: G = p of the kept experts; open-model-atlas
    'All 19 steps': G_i = 2.5 s_i / sum of the selected s), and the output is
    x plus the gate-weighted textbook SwiGLU of exactly those experts."""
    rng = np.random.default_rng(13)
    T, d, N, I, k = 7, 8, 8, 6, 2
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((N, d)).astype(np.float32)
    ex = _rand_experts(rng, N, d, I)
    kw = dict(route_scale=2.5) if gate == "sigmoid" else {}
    cfg = Cfg(n_routed=N, k=k, gate=gate, **kw)
    base = oracle.forward(cfg, x, wr, None, lambda e: ex[e], None)
    # every token keeps its best expert and swaps its second for one it did not pick
    over = base["idx"].copy()
    for t in range(T):
        over[t, 1] = next(e for e in range(N) if e not in base["idx"][t])
    res = oracle.forward(cfg, x, wr, None, lambda e: ex[e], None, idx_override=over)
    x64 = x.astype(np.float64)
    z = torch.from_numpy(x64 @ wr.astype(np.float64).T)
    if gate == "softmax":
        want_g = np.take_along_axis(torch.softmax(z, dim=1).numpy(), over, 1)
    else:
        s_sel = np.take_along_axis(torch.sigmoid(z).numpy(), over, 1)
        want_g = 2.5 * s_sel / s_sel.sum(1, keepdims=True)
    assert np.allclose(res["gates"], want_g, rtol=1e-13, atol=0)
    assert not np.allclose(res["gates"], base["gates"])
    want = x64.copy()
    for t in range(T):
        for j in range(k):
            e = over[t, j]
            want[t] += want_g[t, j] * _torch_swiglu(
                x64[t:t + 1], *(ex[e][n].astype(np.float64) for n in ("w1", "w3", "w2")))[0]
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)


def test_idx_override_keeps_scores():
    rng = np.random.default_rng(10)
    T, d, N = 6, 8, 8
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((N, d)).astype(np.float32)
    ex = _rand_experts(rng, N, d, 4)
    cfg = Cfg(n_routed=N, k=2, gate="sigmoid", route_scale=2.5)
    base = oracle.forward(cfg, x, wr, None, lambda e: ex[e], None)
    same = oracle.forward(cfg, x, wr, None, lambda e: ex[e], None, idx_override=base["idx"])
    assert np.array_equal(base["out"], same["out"])


# ---------------------------------------------------------------- workloads


def test_decode_zipf_bias_empties_about_forty_percent():
    """The decode workload's Zipf bias leaves 102 +- 5 of 256 experts idle."""
    cfg = datagen.get_config("v3_decode")
    inp = datagen.MoEInputs(cfg)
    x64 = oracle.widen(inp.x(), cfg.act_dtype)
    r = oracle.route(cfg, x64, inp.router_w().astype(np.float64), inp.router_b())
    empty = int((r["counts"] == 0).sum())
    assert 97 <= empty <= 107, empty


def test_datagen_streams_are_independent_per_expert():
    cfg = datagen.get_config("deepseekmoe_2b", T=300)
    inp = datagen.MoEInputs(cfg)
    a = inp.expert(5)["w1"]
    stacked = inp.experts_stacked(experts=[4, 5, 6])
    assert np.array_equal(stacked["w1"][1], a)
    x = inp.x()
    assert np.array_equal(inp.x_rows(100, 290), x[100:290])


# ---------------------------------------------------------------- probes 1-2 and balancing


def test_mask_top_brute_force():
    """aiany.app Step 9, probe 1: mask each token's favourite experts and route
    among the rest.  Brute force over all k-subsets of the experts outside the
    token's m best keys; the margin is the m-th minus the (m+1)-th key."""
    rng = np.random.default_rng(21)
    for trial in range(150):
        n = int(rng.integers(3, 12))
        m = int(rng.integers(1, n - 1))
        k = int(rng.integers(1, n - m + 1))
        key = rng.standard_normal(n)
        masked, margin = oracle.exclude_experts(key[None, :], None, m)
        idx, _ = oracle.topk_select(masked, np.ones((1, n), bool), k)
        favourites = set(np.argsort(-key)[:m].tolist())
        rest = [e for e in range(n) if e not in favourites]
        best = max(itertools.combinations(rest, k), key=lambda s: key[list(s)].sum())
        assert set(idx[0].tolist()) == set(best)
        srt = np.sort(key)[::-1]
        assert np.isclose(margin[0], srt[m - 1] - srt[m])


def test_mask_top_grouped_brute_force():
    """Probe 1 under group-limited routing: group scores and the top-k use the
    keys left after masking (brute force on the masked keys)."""
    rng = np.random.default_rng(23)
    for trial in range(100):
        n_groups, gs = 4, 4
        n = n_groups * gs
        m = int(rng.integers(1, 3))
        topk_groups = int(rng.integers(1, n_groups + 1))
        k = int(rng.integers(1, topk_groups * (gs - m) + 1))
        key = rng.standard_normal(n)
        masked, _ = oracle.exclude_experts(key[None, :], None, m)
        allowed, _, _ = oracle.group_limit(masked, n_groups, topk_groups, 2)
        idx, _ = oracle.topk_select(masked, allowed, k)
        fav = np.argsort(-key)[:m]
        kk = key.copy()
        kk[fav] = -1e9  # masked experts can never win a group score or a pick
        assert set(idx[0].tolist()) == _brute_grouped(kk, n_groups, topk_groups, 2, k)
        assert not set(fav.tolist()) & set(idx[0].tolist())


def test_allow_set_and_no_mask_identity():
    rng = np.random.default_rng(22)
    cfg = Cfg(n_routed=16, k=3)
    x = rng.standard_normal((64, 8))
    wr = rng.standard_normal((16, 8))
    base = oracle.route(cfg, x, wr)
    same = oracle.route(cfg, x, wr, allow=np.ones(16, bool), mask_top=0)
    assert np.array_equal(base["idx"], same["idx"]) and np.array_equal(base["gates"], same["gates"])
    allow = np.ones(16, bool)
    allow[[0, 5, 9]] = False
    r = oracle.route(cfg, x, wr, allow=allow)
    assert not np.isin(r["idx"], [0, 5, 9]).any()
    # softmax gates stay the unmasked router's probabilities of the experts kept
    assert np.allclose(r["gates"], np.take_along_axis(base["value"], r["idx"], 1))


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_fewer_picks_is_a_prefix(gate):
    """aiany.app Step 9, probe 2: 4 picks instead of 7 select the first 4 of the
    7 (same order); softmax gates are the same values, sigmoid gates are
    renormalised over the 4 (scale 2.5 over the kept s)."""
    rng = np.random.default_rng(24)
    x = rng.standard_normal((128, 16))
    wr = rng.standard_normal((32, 16))
    kw = dict(n_routed=32, gate=gate, route_scale=1.0 if gate == "softmax" else 2.5)
    if gate == "sigmoid":
        kw.update(n_groups=4, topk_groups=2)
    r7 = oracle.route(Cfg(k=7, **kw), x, wr)
    r4 = oracle.route(Cfg(k=4, **kw), x, wr)
    assert np.array_equal(r4["idx"], r7["idx"][:, :4])
    if gate == "softmax":
        assert np.array_equal(r4["gates"], r7["gates"][:, :4])
    else:
        s4 = np.take_along_axis(r7["value"], r7["idx"][:, :4], 1)
        assert np.allclose(r4["gates"].sum(axis=1), 2.5)
        assert np.allclose(r4["gates"], 2.5 * s4 / s4.sum(axis=1, keepdims=True))


def test_bias_update_direction_and_step():
    """grasp.study lesson 3.2: underloaded experts' biases go up, overloaded ones
    go down, by the fixed step; loads at the mean leave the bias alone.  The
    labels are worked by hand: 12 selections over 6 experts, mean 2."""
    counts = np.array([3, 1, 2, 2, 0, 4])
    label = np.array([-1, +1, 0, 0, +1, -1])  # over, under, at, at, under, over
    b = np.array([0.1, -0.2, 0.05, 0.0, 1.5, -3.0], np.float32)
    nb = oracle.bias_update(b, counts, 12, 0.01)
    assert nb.dtype == np.float32
    d = nb.astype(np.float64) - b.astype(np.float64)
    assert np.array_equal(np.sign(d), label)
    ulp = np.spacing(np.abs(b)).astype(np.float64)
    assert np.all(np.abs(d - 0.01 * label) <= ulp + np.spacing(np.float32(0.01)))
    assert np.array_equal(oracle.bias_update(b, [2] * 6, 12, 0.01), b)


def test_bias_update_balances_routing():
    """The step steers routing towards balance: starting from a bias that favours
    a few experts, repeated route -> count -> update brings the busiest expert
    from over 3x the mean load to within 25% of it."""
    rng = np.random.default_rng(0)
    N, k, T, d = 16, 2, 512, 32
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d)) / np.sqrt(d)
    cfg = Cfg(n_routed=N, k=k, gate="sigmoid", route_scale=1.0)
    b = np.linspace(0.3, -0.3, N).astype(np.float32)
    mean = T * k / N
    first = None
    for _ in range(150):
        c = oracle.route(cfg, x, wr, b)["counts"]
        first = c.max() / mean if first is None else first
        b = oracle.bias_update(b, c, T * k, 0.005)
    last = oracle.route(cfg, x, wr, b)["counts"].max() / mean
    assert first > 3.0 and last < 1.25
