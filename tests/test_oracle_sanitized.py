"""The oracle's C source under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle is built with -fsanitize=address,undefined (gcc, host code only) and
the pins of test_oracle_pins.py (the hand-derived golden values, the brute-force
masked matrix, the closed forms and the twins) run against that build in a
child process with the ASan runtime preloaded. Any out-of-bounds access, use of
freed memory, signed overflow or other undefined behaviour on those inputs stops
the run with a report, and the test fails."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "m3_oracle.c")


def _gcc_lib(name):
    try:
        p = subprocess.run(["gcc", "-print-file-name=" + name], stdout=subprocess.PIPE, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _gcc_lib("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "m3_oracle_asan.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", so, SRC, "-lm"])
        env = dict(os.environ)
        env.update({"M3_ORACLE_LIB": so, "LD_PRELOAD": asan,
                    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
                    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2",
                    "PYTHONDONTWRITEBYTECODE": "1"})
        # every pin except the planted-mistake check, which rebuilds its own
        # (unsanitised) mutants of the source
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-x",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "not planted"],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                           timeout=600)
        out = r.stdout
        assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert r.returncode == 0, out[-4000:]
        assert " passed" in out, out[-2000:]
