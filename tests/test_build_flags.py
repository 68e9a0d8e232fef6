"""The packed-fp32 VALU forms (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32) are
kept out of every kernel: the build passes the target feature that turns them
off, this test shows on a control kernel that the feature does remove them
from the gfx950 code hipcc makes, and that none occurs in the device code of
the built libraries (the ordinary and the checked one).  The device code is
read from each library's own fat binary (clang-offload-bundler +
llvm-objdump): assembly of code built here."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
PACKED = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")
CONTROL = """#include <hip/hip_runtime.h>
typedef float f2 __attribute__((ext_vector_type(2)));
__global__ void k(f2* a, const f2* b, const f2* c) { a[threadIdx.x] = a[threadIdx.x] * b[threadIdx.x] + c[threadIdx.x]; }
"""


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "mixture_experts_ffn_gemm_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _tools():
    need = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in need):
        pytest.skip("ROCm LLVM tools not found")


def test_feature_flag_removes_packed_fp32_from_a_control_kernel():
    _tools()
    b = _build_module()
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "control.hip")
        open(src, "w").write(CONTROL)
        asm = {}
        for name, flags in (("with", b.HIPCC_FLAGS), ("without", [f for f in b.HIPCC_FLAGS if f not in (
                "-Xclang", "-target-feature", "-packed-fp32-ops")])):
            out = os.path.join(tmp, f"{name}.s")
            r = subprocess.run([b.hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", out],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr
            asm[name] = open(out).read()
    assert PACKED.search(asm["without"]), "control: hipcc -O3 packs this float2 FMA by default"
    assert not PACKED.search(asm["with"])


@pytest.mark.parametrize("name", ["libmoe.so", "libmoe_checked.so"])
def test_built_library_has_no_packed_fp32(name):
    _tools()
    lib = os.path.join(ROOT, "mixture_experts_ffn_gemm_amd", name)
    if not os.path.exists(lib):
        pytest.skip(f"{name} not built")
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib],
                       check=True)
        data = open(fat, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = [m.start() for m in re.finditer(re.escape(magic), data)]
        assert starts, "no offload bundle in the library"
        mfma = 0
        for i, s0 in enumerate(starts):
            end = starts[i + 1] if i + 1 < len(starts) else len(data)
            part = os.path.join(tmp, f"b{i}.bin")
            open(part, "wb").write(data[s0:end])
            co = os.path.join(tmp, f"b{i}.co")
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                            f"--output={co}"], check=True)
            dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", co],
                                 capture_output=True, text=True, check=True).stdout
            bad = PACKED.findall(dis)
            assert not bad, f"bundle {i}: {len(bad)} packed fp32 instructions"
            mfma += len(re.findall(r"\bv_mfma_", dis))
        assert mfma > 0  # the disassembly really is the kernels' code
