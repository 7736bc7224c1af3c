"""The library's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer -- CPU only.

The HIP library is rebuilt with the sanitizers on its host pass only (each
flag behind -Xarch_host; the gfx950 code is built as usual) into a temporary
directory, and the C-ABI tests run against it in a child process that preloads
clang's ASan runtime.  Those tests reach every entry point's argument,
alignment and workspace checks and the workspace layout arithmetic, and no
kernel launch.
"""
import glob
import os
import subprocess
import sys

import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]

CHILD = r"""
import sys
import moe_layer_gating_amd as moe
moe.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py",
                      "-k", "not bench_refuses"]))
"""


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_checks_under_asan_ubsan():
    import moe_layer_gating_amd._build as b

    rt = _asan_runtime()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if rt is None or not os.path.exists(hipcc):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        san_lib = os.path.join(d, "libmoe_gfx950_san.so")
        subprocess.run([hipcc, *b.HIPCC_FLAGS, *HOST_SAN, "-I", b.INCLUDE, "-o", san_lib,
                        *b.sources()], check=True, capture_output=True, timeout=900)
        env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-c", CHILD, san_lib], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
