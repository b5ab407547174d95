"""The C-ABI front end (argument validation, workspace layout, error
reporting) built with host-side AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the ABI tests run clean against the instrumented library, and the
instrumentation does stop a planted stack overrun in a copy of the front end,
so a clean run means something.  The device code is the regular build's; only
dsa_api.cpp is instrumented, for the host (-Xarch_host)."""
import glob
import os
import subprocess
import sys

import pytest

import long_context_sparse_14_amd as dsa
from long_context_sparse_14_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="CPU-only: the ABI tests pass fake device pointers")


def _asan_runtime():
    rt = sorted(glob.glob(os.path.join(os.path.dirname(B.hipcc()), "..", "llvm", "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so")))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return os.path.realpath(rt[-1])


def _build(tmp, api_source):
    """libdsa with api_source instrumented, linked with the regular build's other objects."""
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "dsa_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build_library()
    api_o = os.path.join(tmp, "dsa_api_san.o")
    cmd = [B.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}", "-I", B.INCLUDE, "-I", B.CSRC,
           "-x", "hip"] + HOST_SAN + ["-c", api_source, "-o", api_o]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lib = os.path.join(tmp, "libdsa_san.so")
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib] + objs + [api_o] +
                   ["-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan"],
                   check=True, capture_output=True, timeout=600)
    return lib


def _env(lib):
    env = dict(os.environ)
    env.update(DSA_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_abi_tests_run_clean_under_asan_and_ubsan(tmp_path):
    lib = _build(str(tmp_path), os.path.join(B.CSRC, "dsa_api.cpp"))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and "passed" in res.stdout, res.stdout[-3000:] + res.stderr[-3000:]
    assert "skipped" not in res.stdout.splitlines()[-1], res.stdout[-500:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """A copy of the front end whose error formatting is handed the size of
    the 512-byte message buffer for a 16-byte stack buffer: the first
    rejected call must stop in the instrumented build."""
    with open(os.path.join(B.CSRC, "dsa_api.cpp")) as f:
        src = f.read()
    old = "  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);\n"
    assert src.count(old) == 1
    bad = tmp_path / "dsa_api_overrun.cpp"
    bad.write_text(src.replace(old, "  char tmp[16];\n  vsnprintf(tmp, sizeof(g_last_error), fmt, ap);\n"
                                    "  memcpy(g_last_error, tmp, sizeof(tmp));\n"))
    lib = _build(str(tmp_path), str(bad))
    code = ("import long_context_sparse_14_amd as dsa\n"
            "rc = dsa.library().dsa_calib_stream(None, None, 64, None)\n"   # rejected: src is NULL
            "print('returned', rc)\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib), capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, res.stdout[-500:] + res.stderr[-2000:]
