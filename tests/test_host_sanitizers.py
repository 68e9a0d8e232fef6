"""The host side of the library (argument validation, workspace layout, expert
masks, the no-allocation entry point's size check: api.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer, and the C-ABI checks of
test_abi_cpu.py run against that build in a child process.  Only host code
is instrumented (each -fsanitize flag is passed to the host compilation
alone); the kernels are built as usual.  No GPU is needed: every call the
ABI checks make fails validation before any launch."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_ONLY = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "mixture_experts_ffn_gemm_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_code_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime not found")

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        san = HOST_ONLY if src.endswith("api.cpp") else []
        cmd = [cc, *(["-x", "hip"] if src.endswith(".cpp") else []), *b.HIPCC_FLAGS, *san,
               "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, b.sources()))
    lib = str(tmp_path / "libmoe_sanitized.so")
    r = subprocess.run([cc, "-shared", f"--offload-arch={b.ARCH}", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", lib, *objs,
                        *b.LINK_LIBS],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_PRELOAD=rt[-1], MOE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the sanitized build is the one loaded, with the ASan runtime
    probe = ("import mixture_experts_ffn_gemm_amd as m, sys; maps = open('/proc/self/maps').read(); "
             "sys.exit(0 if m.LIB_PATH.endswith('libmoe_sanitized.so') and 'libmoe_sanitized.so' in maps "
             "and 'libclang_rt.asan' in maps else 3)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
