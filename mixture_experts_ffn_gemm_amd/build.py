"""Build libmoe.so (gfx950) from csrc/ with hipcc, in-tree.

    python mixture_experts_ffn_gemm_amd/build.py        # or __graft_entry__.build()

Every .hip / .cpp file under csrc/ is compiled to an object in _build/ at the
repository root and linked into mixture_experts_ffn_gemm_amd/libmoe.so.  The
checked library, libmoe_checked.so (the same sources with MOE_DEVICE_CHECKS=1:
kernels record index-range violations, entry points report them), is built
from objects in _build/checked/.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
LIB_CHECKED = os.path.join(PKG, "libmoe_checked.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# roctx ranges around the forward's stages (rocprofiler-sdk's marker library)
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, checked: bool = False) -> str:
    bdir = os.path.join(BUILD, "checked") if checked else BUILD
    out = LIB_CHECKED if checked else LIB
    extra = ["-DMOE_DEVICE_CHECKS=1"] if checked else []
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [cc, *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LINK_LIBS]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, checked=True))
