"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C source is built with ``-fsanitize=address,undefined`` (host
code only: the oracle never touches a GPU) and the six pin files run against
that build in a subprocess, with the sanitizer runtime preloaded into the
Python interpreter that loads it through ctypes.  Any out-of-bounds access,
use after free or undefined behaviour (shift, overflow, misaligned access)
aborts the run; every pin must still pass.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PIN_FILES = ["test_oracle_formats.py", "test_oracle_router.py", "test_oracle_ffn.py",
             "test_oracle_mx.py", "test_oracle_tail.py", "test_oracle_fp8.py"]


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_clean_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call([
        "gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
        "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
        "-shared", "-fPIC", "-o", str(so), SRC, "-lm"])
    preload = [asan]
    ubsan = _runtime("libubsan.so")
    if ubsan:
        preload.append(ubsan)
    env = dict(os.environ, MOE_ORACLE_LIB=str(so), LD_PRELOAD=":".join(preload),
               # leaks of the Python interpreter itself are not the oracle's
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    pins = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider"] + pins,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, "sanitized oracle run failed:\n" + report
    for marker in ("ERROR: AddressSanitizer", "runtime error:"):
        assert marker not in r.stderr, "sanitizer report:\n" + report
