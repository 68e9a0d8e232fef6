"""The checked library (libmoe_checked.so: the same sources built with
MOE_DEVICE_CHECKS=1) on the GPU.  With valid inputs every call returns MOE_OK
and the same bits as the ordinary library.  An index outside its range is
recorded by the kernel that reads it, replaced by a safe one before any
access, and reported by the call as MOE_ERR_DEVICE_CHECK naming the check.
Out-of-range indices are only ever given to the checked library."""
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
    import mixture_experts_ffn_gemm_amd as m  # fails loudly without the built library
    return m


@pytest.fixture(scope="module")
def checked(lib):
    return lib._lib.load_checked()


class using:
    """Route the binding's calls to another build of the library."""

    def __init__(self, lib, handle):
        self.mod, self.handle = lib._lib, handle

    def __enter__(self):
        self.old = self.mod.LIB
        self.mod.LIB = self.handle

    def __exit__(self, *exc):
        self.mod.LIB = self.old


# small forwards through every kernel family: bf16 persistent GEMMs (V3-shaped
# prefill, few rows per expert), fp8 weight streaming (decode), fp8 persistent
# GEMMs (many rows per expert), fp32 MFMA GEMMs (GShard)
CASES = {
    "v3_prefill": dict(T=500, d=1024, inter=256),
    "v3_decode": dict(d=1024, inter=512),
    "fp8_prefill": dict(T=600, d=1024, inter=256, n_routed=32, w_dtype="fp8",
                        w_block=datagen.FP8_BLOCK),
    "gshard_fp32": dict(),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("side", [False, True])
def test_checked_forward_is_clean_and_bitwise_equal(lib, checked, case, side):
    name = "v3_prefill" if case == "fp8_prefill" else case
    cfg = datagen.get_config(name, **CASES[case])
    say(f"[checked] forward {case} T={cfg.T} d={cfg.d} w={cfg.w_dtype} side stream={side}")
    dev = upload(datagen.MoEInputs(cfg))
    c = lib.config_from(cfg)

    def run():
        r = lib.forward(c, dev["x"], dev["w_r"], dev["b"], dev["experts"], dev["shared"],
                        want_routing=True, side_stream=torch.cuda.Stream() if side else None)
        torch.cuda.synchronize()
        return r

    want = run()
    with using(lib, checked):
        got = run()
    for a, b in zip(want, got):
        assert torch.equal(a, b)


def _expect_check(lib, fn, words):
    with pytest.raises(lib.MoeError) as e:
        fn()
    assert e.value.status == lib._lib.MOE_ERR_DEVICE_CHECK
    msg = str(e.value)
    for w in words:
        assert w in msg, msg


def test_checked_permute_reports_out_of_range_ids(lib, checked):
    T, k, N = 300, 6, 64
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    cfg = datagen.get_config("v3_prefill", T=T, k=k, n_routed=N, n_groups=1, topk_groups=1,
                             d=256, inter=128, n_shared=0)
    c = lib.config_from(cfg)
    good = torch.from_numpy(idx).cuda()
    with using(lib, checked):
        lib.permute(c, good)  # valid ids: MOE_OK
        torch.cuda.synchronize()
    idx[3, 2], idx[100, 0] = N + 4, -2
    bad = torch.from_numpy(idx).cuda()
    # the ordinary library clamps such ids (its documented contract) and says nothing
    lib.permute(c, bad)
    torch.cuda.synchronize()
    with using(lib, checked):
        _expect_check(lib, lambda: lib.permute(c, bad), ["expert id"])
        lib.permute(c, good)  # the flags were cleared by the report
        torch.cuda.synchronize()


def test_checked_combine_reports_out_of_range_slots(lib, checked):
    T, k, d = 64, 4, 256
    cfg = datagen.get_config("v3_prefill", T=T, k=k, d=d, inter=128, n_shared=0, act_dtype="bf16",
                             out_dtype="f32")
    c = lib.config_from(cfg)
    rng = np.random.default_rng(6)
    y = torch.from_numpy(rng.standard_normal((T * k, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    slot = rng.permutation(T * k).astype(np.int32)
    gate = torch.from_numpy(rng.uniform(0, 1, (T, k)).astype(np.float32)).cuda()
    with using(lib, checked):
        lib.combine(c, y, torch.from_numpy(slot).cuda(), gate)
        torch.cuda.synchronize()
        slot[7] = T * k + 9
        _expect_check(lib, lambda: lib.combine(c, y, torch.from_numpy(slot).cuda(), gate),
                      ["combine slot"])


def test_checked_expert_ffn_reports_out_of_range_rows(lib, checked):
    T, d, I, E = 300, 256, 128, 8
    cfg = datagen.get_config("v3_prefill", T=T, d=d, inter=I, n_routed=E, n_groups=1,
                             topk_groups=1, k=2, n_shared=0)
    c = lib.config_from(cfg)
    rng = np.random.default_rng(7)
    counts = np.array([0, 1, 255, 256, 40, 0, 0, 48], np.int64)  # T*k = 600 rows in all
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    rows = int(counts.sum())
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    w = [torch.from_numpy((rng.standard_normal(s) * 0.05).astype(np.float32)).to(torch.bfloat16).cuda()
         for s in ((E, I, d), (E, I, d), (E, d, I))]
    ri = rng.integers(0, T, rows).astype(np.int32)
    want = lib.expert_ffn(c, E, off, rows, x, *w, row_index=torch.from_numpy(ri).cuda())
    torch.cuda.synchronize()
    with using(lib, checked):
        got = lib.expert_ffn(c, E, off, rows, x, *w, row_index=torch.from_numpy(ri).cuda())
        torch.cuda.synchronize()
        assert torch.equal(want, got)
        ri[5], ri[rows - 1] = T + 3, 1 << 24
        _expect_check(lib, lambda: lib.expert_ffn(c, E, off, rows, x, *w,
                                                  row_index=torch.from_numpy(ri).cuda()),
                      ["activation row"])
