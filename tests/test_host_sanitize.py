"""The library's host code (rtl_api.cpp: argument validation, error reporting, dispatch)
built with AddressSanitizer and UndefinedBehaviorSanitizer and linked with the other
objects of the in-tree build, then the C ABI tests (tests/test_abi.py) run against it in a
subprocess with the sanitizer runtime preloaded.  CPU only: every call there fails
validation or finds no GPU, so no kernel runs."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "activation_sparse_gemm_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all"]


def _runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None, reason="needs hipcc and its ASan runtime")
def test_abi_under_asan_ubsan(tmp_path):
    objs = [os.path.join(PKG, "_build", n + ".o") for n in ("sparsify", "prep_bf16", "gemm_bf16", "gemm_fp8",
                                                          "fp32_path", "noalloc", "mlp_bf16")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("build the library first (activation_sparse_gemm_amd/build.py)")
    api = tmp_path / "rtl_api.o"
    so = tmp_path / "librtl_sanitized.so"
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", *SAN,
                    "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(PKG, "csrc", "rtl_api.cpp"), "-o",
                    str(api)], check=True, capture_output=True)
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", str(api), *objs, "-o", str(so)], check=True,
                   capture_output=True)
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", RTL_LIBRARY=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
