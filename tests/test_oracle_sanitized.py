"""The oracle's pin tests again, with the oracle built under AddressSanitizer
and UndefinedBehaviorSanitizer (out-of-bounds or use-after-free accesses,
signed overflow, bad shifts, misaligned loads abort the run) -- CPU only.

The child process preloads gcc's ASan runtime (the Python interpreter is
not instrumented) and loads oracle/libmoe_oracle_san.so through
MOE_ORACLE_SANITIZE=1.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_codecs.py", "tests/test_oracle_routing.py",
             "tests/test_oracle_ffn.py", "tests/test_oracle_rope.py"]


def _asan_runtime():
    try:
        out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.build(sanitize=True)
    env = dict(os.environ, MOE_ORACLE_SANITIZE="1", LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + PIN_TESTS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
