"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and streams; nothing here
computes.  Importing this module loads the library and fails loudly if it
has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, c_char_p, POINTER

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_LIBRARY may name another build of the same sources
# (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(PKG, "libmoe.so")
# the same sources built with MOE_DEVICE_CHECKS=1 (kernels record index-range
# violations; every call synchronises and reports them as MOE_ERR_DEVICE_CHECK)
LIB_CHECKED_PATH = os.path.join(PKG, "libmoe_checked.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_DEVICE_CHECK = -5
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
GATES = {"softmax": 0, "sigmoid": 1}

# every symbol include/moe.h declares
EXPORTS = ["moe_status_string", "moe_last_error", "moe_version", "moe_workspace_size",
           "moe_router", "moe_router_masked", "moe_bias_update", "moe_permute", "moe_expert_ffn",
           "moe_combine", "moe_forward", "moe_forward_timed", "moe_forward_noalloc"]


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int32), ("n_routed", c_int32), ("n_shared", c_int32),
                ("inter", c_int32), ("k", c_int32), ("n_groups", c_int32),
                ("topk_groups", c_int32), ("group_topn", c_int32), ("gate", c_int32),
                ("route_scale", c_float), ("act_dtype", c_int32), ("w_dtype", c_int32),
                ("out_dtype", c_int32), ("w_block", c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status_string(status)}: {msg}")
        self.status = status


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python mixture_experts_ffn_gemm_amd/build.py`")
    lib = ctypes.CDLL(path)
    P = c_void_p
    lib.moe_status_string.restype = c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_last_error.restype = c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_version.restype = c_char_p
    lib.moe_version.argtypes = []
    lib.moe_workspace_size.restype = c_size_t
    lib.moe_workspace_size.argtypes = [POINTER(MoeConfig)]
    lib.moe_router.restype = ctypes.c_int
    lib.moe_router.argtypes = [POINTER(MoeConfig), P, P, P, P, P, P, P, c_size_t, P]
    lib.moe_router_masked.restype = ctypes.c_int
    lib.moe_router_masked.argtypes = [POINTER(MoeConfig), P, P, P, P, c_int32, P, P, P, P, c_size_t,
                                      P]
    lib.moe_bias_update.restype = ctypes.c_int
    lib.moe_bias_update.argtypes = [POINTER(MoeConfig), P, P, c_float, P]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_permute.argtypes = [POINTER(MoeConfig), P, P, P, P, P, P, P, P, c_size_t, P]
    lib.moe_expert_ffn.restype = ctypes.c_int
    lib.moe_expert_ffn.argtypes = [POINTER(MoeConfig), c_int32, P, c_int64, c_int32, P, P, P, P, P,
                                   P, P, P, P, P, c_size_t, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [POINTER(MoeConfig), P, P, P, P, P, P, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [POINTER(MoeConfig)] + [P] * 20 + [c_size_t, P, P]
    lib.moe_forward_timed.restype = ctypes.c_int
    lib.moe_forward_timed.argtypes = [POINTER(MoeConfig)] + [P] * 20 + [c_size_t, P, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [POINTER(MoeConfig)] + [P] * 19 + [P, P]
    return lib


# size of moe_forward_noalloc's static per-GPU scratch array (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


LIB = _load()


def load_checked():
    """The checked library (libmoe_checked.so), loaded beside LIB with the same
    signatures; the binding's functions use it while ``_lib.LIB`` is set to it."""
    return _load(LIB_CHECKED_PATH)


def status_string(status: int) -> str:
    return LIB.moe_status_string(status).decode()


def last_error() -> str:
    return LIB.moe_last_error().decode()


def version() -> str:
    return LIB.moe_version().decode()


def check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, last_error())


def make_config(T, d, n_routed, n_shared, inter, k, n_groups=1, topk_groups=1, group_topn=2,
                gate="softmax", route_scale=1.0, act_dtype="bf16", w_dtype="bf16",
                out_dtype="f32", w_block=0) -> MoeConfig:
    return MoeConfig(T=T, d=d, n_routed=n_routed, n_shared=n_shared, inter=inter, k=k,
                     n_groups=n_groups, topk_groups=topk_groups, group_topn=group_topn,
                     gate=GATES[gate], route_scale=route_scale, act_dtype=DTYPES[act_dtype],
                     w_dtype=DTYPES[w_dtype], out_dtype=DTYPES[out_dtype], w_block=w_block)


def config_from(c) -> MoeConfig:
    """MoeConfig from any object with the layer's fields (e.g. datagen.MoEConfig)."""
    return make_config(c.T, c.d, c.n_routed, c.n_shared, c.inter, c.k, c.n_groups, c.topk_groups,
                       c.group_topn, c.gate, c.route_scale, c.act_dtype, c.w_dtype, c.out_dtype,
                       c.w_block)


def workspace_size(cfg: MoeConfig) -> int:
    return int(LIB.moe_workspace_size(ctypes.byref(cfg)))
