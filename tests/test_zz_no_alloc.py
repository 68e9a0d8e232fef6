"""moe_forward_noalloc (the forward on the library's static per-GPU scratch
array, for callers that cannot allocate) against moe_forward with a caller
workspace: bitwise-equal outputs and routing on two calls in a row, the
second with fewer tokens, for the fp8 decode step (weight-streaming GEMMs)
and a small bf16 prefill (persistent GEMMs, whose padding rows read the
zeroed rows of the scratch)."""
import numpy as np
import pytest
import torch

import datagen
from datagen.device import upload
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import mixture_experts_ffn_gemm_amd as m
    return m


@pytest.mark.parametrize("name,T0,T1,over", [
    ("v3_decode", 64, 16, {}),
    ("v3_prefill", 600, 250, dict(d=1024, inter=256)),
])
def test_noalloc_matches_forward(lib, name, T0, T1, over):
    full = datagen.get_config(name, T=T0, **over)
    assert lib.workspace_size(lib.config_from(full)) <= lib.NOALLOC_SCRATCH_BYTES
    dev = upload(datagen.MoEInputs(full))
    side = torch.cuda.Stream()
    for T in (T0, T1):
        cfg = full.replace(T=T)
        say(f"[noalloc] {name} T={T} d={cfg.d} I={cfg.inter} w={cfg.w_dtype}")
        c = lib.config_from(cfg)
        x = dev["x"][:T].contiguous()
        args = (c, x, dev["w_r"], dev["b"], dev["experts"], dev["shared"])
        ref = lib.forward(*args, want_routing=True, side_stream=side)
        torch.cuda.synchronize()
        got = lib.forward_noalloc(*args, want_routing=True, side_stream=side)
        torch.cuda.synchronize()
        for a, b, what in zip(ref, got, ("out", "topk_idx", "topk_gate", "counts")):
            assert torch.equal(a, b), f"{what} differs at T={T}"
        one = lib.forward_noalloc(*args)  # one stream: the shared expert folded in
        torch.cuda.synchronize()
        assert torch.equal(one, ref[0])
        say(f"   equal to moe_forward (two streams and one), out RMS "
            f"{float(ref[0].float().pow(2).mean().sqrt()):.3f}")
