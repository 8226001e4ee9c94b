"""The C-ABI validation layer (qlin_api.hip) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer, linked with stub launchers
(tests/hostcheck/stub_launchers.cpp) instead of the kernels, and driven from a
child process on the CPU: boundary cases, a 20000-call random sweep of every
entry point, and a planted out-of-bounds read as a positive control that the
sanitizer is live.  Built with g++ (host code only)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "hostcheck")


def _asan_runtime():
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    p = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("g++ with AddressSanitizer is not installed")
    out = str(tmp_path_factory.mktemp("hostcheck") / "libqlin_hostcheck.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-fPIC", "-shared", "-x", "c++", os.path.join(ROOT, "quantized_linear_layers_token_amd", "csrc", "qlin_api.hip"),
           "-x", "c++", os.path.join(HC, "stub_launchers.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out, asan


def _run(lib, asan, *extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + ((" " + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([sys.executable, os.path.join(HC, "validation_driver.py"), lib, *extra],
                          capture_output=True, text=True, env=env, timeout=600)


def test_validation_layer_clean_under_asan_and_ubsan(sanitized_lib):
    r = _run(*sanitized_lib)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "no sanitizer report" in r.stdout


def test_planted_overflow_is_caught(sanitized_lib):
    # the library reads segments[0 .. nseg): announcing two over a one-entry
    # array must be reported, or the clean run above proves nothing
    r = _run(*sanitized_lib, "--planted-overflow")
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]
