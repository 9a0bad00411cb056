"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C source is built with -fsanitize=address,undefined (every
undefined-behaviour report fatal) next to its usual flags, and the three pin
files run against that build in a child process through the oracle's library
override (MOONEP_ORACLE_LIB), with the sanitizer runtime preloaded into the
Python interpreter that loads it. Any out-of-bounds access, use after free or
undefined operation in the oracle's loops ends the child with an error, so the
pins passing here means they also passed without a sanitizer report. Leak
detection is off: the interpreter itself is not built with the sanitizer. The
child runs its OpenMP loops on two threads.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moonep_oracle.c")
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_bounded_pins.py",
             "tests/test_oracle_backward_pins.py", "tests/test_oracle_threads.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_on_a_sanitized_oracle(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    so = str(tmp_path / "libmoonep_oracle_san.so")
    subprocess.check_call(["gcc"] + oracle.CFLAGS + [
        "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all", "-o", so, SRC, "-lm"])
    env = dict(os.environ, MOONEP_ORACLE_LIB=so, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2",
               PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not 4-4-1-2"] + PIN_FILES
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in out, out
