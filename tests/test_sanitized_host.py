"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The block manager and scheduler (csrc/scheduler.cpp), the host side of the
library's entry points (argument checks, plans, pkv_validate_step) and the
oracle (oracle/oracle.c) are built with -fsanitize=address,undefined
(paged_kv_decode_append_amd/build.py --sanitize, oracle.build(sanitize=True)),
and the CPU tests of those parts -- tests/test_scheduler.py,
tests/test_abi.py and tests/test_oracle.py -- run against that build in a
child process with the sanitizer runtime preloaded; any report aborts the
child.  A planted out-of-bounds read through pkv_validate_step (a block
table shorter than its declared width) must be reported, which shows the
sanitizers are live in that process.  No GPU: nothing here launches a
kernel.  CPU only.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(ROOT, "paged_kv_decode_append_amd"))
import build as pkv_build  # noqa: E402  (the build script, not the package)

import oracle  # noqa: E402


@pytest.fixture(scope="module")
def sanitized_env(tmp_path_factory):
    runtime = pkv_build.san_runtime()
    if runtime is None or not os.path.exists(pkv_build.HIPCC) or not os.path.exists(pkv_build.SAN_CXX):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    lib = pkv_build.build(sanitize=True)
    olib = oracle.build(out=str(tmp_path_factory.mktemp("san") / "liboracle.so"), sanitize=True)
    return dict(os.environ, PKV_LIBRARY=lib, ORACLE_LIBRARY=olib, LD_PRELOAD=runtime,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def test_scheduler_abi_and_oracle_tests_pass_under_sanitizers(sanitized_env):
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
         os.path.join(HERE, "test_scheduler.py"), os.path.join(HERE, "test_abi.py"),
         os.path.join(HERE, "test_oracle.py")],
        cwd=ROOT, env=sanitized_env, capture_output=True, text=True, timeout=900)
    print(res.stdout[-1500:])
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout and "failed" not in res.stdout


PLANTED = r"""
import ctypes, numpy as np, paged_kv_decode_append_amd as pkv
assert pkv.LIB_PATH.endswith("_build/sanitize/libpkv.so"), pkv.LIB_PATH
width = 64                                  # declared table width ...
bt = np.zeros(8, dtype=np.int32)            # ... but a row of 8 entries
ctx = np.array([width * 16], dtype=np.int32)
bad_what, bad_idx = ctypes.c_int32(0), ctypes.c_int64(0)
pkv.lib.pkv_validate_step(bt.ctypes.data, width, ctx.ctypes.data, None, 1, 1, 1 << 20, 16,
                          None, 1, int(ctx[0]), 1, ctypes.byref(bad_what), ctypes.byref(bad_idx))
print("no report")
"""


def test_a_planted_overflow_is_reported(sanitized_env):
    res = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=sanitized_env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, \
        res.stdout[-2000:] + res.stderr[-4000:]
