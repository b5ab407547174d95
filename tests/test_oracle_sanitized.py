"""The C++ oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every pin runs clean on the instrumented build, and the
instrumented build does catch an out-of-bounds write planted in a copy of the
oracle, so a clean run means something."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _env(lib):
    rt = [_runtime("libasan.so"), _runtime("libubsan.so")]
    if None in rt:
        pytest.skip("the gcc sanitizer runtimes are not installed")
    env = dict(os.environ)
    env.update(DSA_ORACLE_LIB=lib, LD_PRELOAD=":".join(rt), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", DSA_ORACLE_THREADS="4")
    return env


def test_pins_run_clean_under_asan_and_ubsan(tmp_path):
    lib = oracle.build_library(force=True, out=str(tmp_path / "liboracle_san.so"), extra_flags=SAN_FLAGS)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and "passed" in res.stdout, res.stdout[-3000:] + res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """A copy of the oracle whose visible-key count ignores the cache length
    writes past the score buffer: the instrumented build must stop on it."""
    with open(oracle.SOURCE) as f:
        src = f.read()
    old = "return std::min(N, p1 / m);"
    assert src.count(old) == 1
    bad = tmp_path / "overrun.cpp"
    bad.write_text(src.replace(old, "return p1 / m;"))
    lib = oracle.build_library(force=True, source=str(bad), out=str(tmp_path / "liboverrun_san.so"),
                               extra_flags=SAN_FLAGS)
    code = ("import numpy as np, oracle\n"
            "q = np.ones((1, 8, 1, 4), np.float32); k = np.ones((1, 2, 4), np.float32); w = np.ones((1, 8, 1), np.float32)\n"
            "oracle.index_scores_batch(q, k, w, [(0, 7)], 0)\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib), capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, res.stderr[-2000:]
