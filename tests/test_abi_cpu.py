"""Host-side checks of the C ABI: the library loads, exports every symbol
include/moe.h declares, sizes its workspace, and rejects bad arguments
before launching anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    import mixture_experts_ffn_gemm_amd as m
    return m


def test_header_symbols_exported(m):
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    declared = set(re.findall(r"^\s*(?:const char\*|size_t|int)\s+(moe_\w+)\s*\(", hdr, re.M))
    assert declared == set(m.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    assert declared <= exported, declared - exported
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name)


def test_status_strings(m):
    assert m.status_string(0) == "MOE_OK"
    assert m.status_string(-3) == "MOE_ERR_WORKSPACE"
    assert m.status_string(-5) == "MOE_ERR_DEVICE_CHECK"
    assert "gfx950" in m.version()


def test_checked_library_loads_and_exports(m):
    """The checked build (MOE_DEVICE_CHECKS=1) exports the same symbols and
    validates arguments on the host the same way."""
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    declared = set(re.findall(r"^\s*(?:const char\*|size_t|int)\s+(moe_\w+)\s*\(", hdr, re.M))
    path = m._lib.LIB_CHECKED_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert declared <= set(re.findall(r" T (moe_\w+)", out))
    lib = m._lib.load_checked()
    assert lib.moe_status_string(-5).decode() == "MOE_ERR_DEVICE_CHECK"
    cfg = m.config_from(datagen.get_config("v3_prefill", T=64))
    assert lib.moe_workspace_size(ctypes.byref(cfg)) == m.workspace_size(cfg)
    bad = m.config_from(datagen.get_config("v3_prefill", T=64))
    bad.k = 0
    assert lib.moe_workspace_size(ctypes.byref(bad)) == 0


def test_workspace_sizes(m):
    for name in datagen.CONFIG_ORDER:
        c = m.config_from(datagen.get_config(name))
        assert m.workspace_size(c) > 0
    big = m.workspace_size(m.config_from(datagen.get_config("v3_prefill")))
    # holds at least the routed H [T*k, I] and Y [T*k, d] bf16 buffers
    assert big >= 16384 * 8 * (2048 + 7168) * 2


@pytest.mark.parametrize("field,value", [
    ("k", 0), ("k", 300), ("n_routed", 0), ("n_routed", 512), ("n_groups", 3),
    ("topk_groups", 9), ("group_topn", 40), ("d", 100), ("inter", 200), ("act_dtype", 2),
    ("w_block", 64), ("gate", 5), ("T", -1), ("out_dtype", 2)])
def test_invalid_configs_rejected(m, field, value):
    c = m.config_from(datagen.get_config("v3_prefill"))
    setattr(c, field, value)
    assert m.workspace_size(c) == 0
    st = m._lib.LIB.moe_router(c, None, None, None, None, None, None, None, 0, None)
    assert st in (-1, -2), st
    assert m.last_error()


def test_k_beyond_kept_groups_rejected(m):
    c = m.config_from(datagen.get_config("v3_prefill"))
    c.topk_groups, c.k = 1, 33  # one group of 32 experts cannot supply 33 picks
    st = m._lib.LIB.moe_router(c, None, None, None, None, None, None, None, 0, None)
    assert st == -1 and "k exceeds" in m.last_error()


def test_null_pointers_and_small_workspace_rejected(m):
    c = m.config_from(datagen.get_config("deepseekmoe_2b"))
    L = m._lib.LIB
    assert L.moe_router(c, None, None, None, None, None, None, None, 0, None) == -1
    # non-null (never dereferenced) pointers but no workspace
    p = 0x1000
    assert L.moe_router(c, p, p, None, p, p, None, None, 0, None) == -3
    assert "workspace" in m.last_error()
    assert L.moe_forward(c, *([None] * 20), 0, None, None) == -1
    assert L.moe_expert_ffn(c, 0, p, 10, 0, p, None, p, p, p, None, None, None, p, p, 1 << 40, None) == -1
    assert L.moe_expert_ffn(c, 2, p, 10, 0, p, None, p, p, p, p, p, p, p, p, 1 << 40, None) == -1  # scales on bf16
    assert L.moe_combine(c, None, None, None, None, None, None, None) == -1


def test_empty_batch_is_a_no_op(m):
    c = m.config_from(datagen.get_config("v3_prefill"))
    c.T = 0
    assert m.workspace_size(c) > 0
    c.T, c.d = 1, 128
    assert m.workspace_size(c) > 0
    c.T, c.d = 0, 7168
    assert m._lib.LIB.moe_router(c, None, None, None, None, None, None, None, 0, None) == 0
    assert m._lib.LIB.moe_combine(c, None, None, None, None, None, None, None) == 0


def test_router_masked_rejects_exclusions_that_leave_too_few(m):
    L = m._lib.LIB
    c = m.config_from(datagen.get_config("deepseekmoe_2b"))  # 63 experts, k = 7, ungrouped
    allow = (ctypes.c_uint8 * 63)(*([1] * 8 + [0] * 55))     # 8 allowed experts
    p = 0x1000
    # 8 allowed - mask_top 2 < k = 7
    assert L.moe_router_masked(c, p, p, None, ctypes.cast(allow, ctypes.c_void_p), 2, p, p, None,
                               None, 0, None) == -1
    assert "fewer than k" in m.last_error()
    assert L.moe_router_masked(c, p, p, None, None, -1, p, p, None, None, 0, None) == -1
    v3 = m.config_from(datagen.get_config("v3_prefill"))    # 8 groups of 32, top-2 group score
    allow = (ctypes.c_uint8 * 256)(*([1] * 224 + [0] * 30 + [1] * 2))  # last group keeps 2
    assert L.moe_router_masked(v3, p, p, None, ctypes.cast(allow, ctypes.c_void_p), 1, p, p, None,
                               None, 0, None) == -1
    assert "group_topn + mask_top" in m.last_error()
    # valid exclusions with no workspace reach the workspace check (nothing is launched)
    assert L.moe_router_masked(v3, p, p, None, None, 8, p, p, None, None, 0, None) == -3


def test_bias_update_argument_checks(m):
    L = m._lib.LIB
    c = m.config_from(datagen.get_config("v3_prefill"))
    p = 0x1000
    assert L.moe_bias_update(c, None, p, 0.001, None) == -1
    assert L.moe_bias_update(c, p, None, 0.001, None) == -1
    assert L.moe_bias_update(c, p, p, float("nan"), None) == -1
    assert L.moe_bias_update(c, p, p, -1.0, None) == -1


def test_noalloc_forward_rejects_configs_beyond_its_scratch(m):
    """moe_forward_noalloc refuses, before touching the device, a config whose
    workspace exceeds its static scratch array; the V3-shaped decode step fits."""
    L = m._lib.LIB
    dec = m.config_from(datagen.get_config("v3_decode"))
    assert 0 < m.workspace_size(dec) <= m.NOALLOC_SCRATCH_BYTES
    big = m.config_from(datagen.get_config("v3_prefill"))
    assert m.workspace_size(big) > m.NOALLOC_SCRATCH_BYTES
    p = 0x1000
    assert L.moe_forward_noalloc(big, *([p] * 19), None, None) == -3
    assert "moe_forward_noalloc has" in m.last_error()
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", hdr)
    assert m.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert L.moe_forward_noalloc(None, *([None] * 19), None, None) == -1
