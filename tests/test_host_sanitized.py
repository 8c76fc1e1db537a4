"""The library's host code (argument checks, workspace sizing, dispatch, the
RoPE table) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
against the stand-in runtime of host_asan/stubs.cpp, then driven by
test_abi.py, host_asan/check_dispatch.py and host_asan/fuzz_args.py (randomised
arguments for every entry point) in a child process that has the
sanitizer runtime preloaded.  Any sanitizer report fails the test.  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "exact_scaled_dot_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "libattn_host_san.so")


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_under_asan_and_ubsan():
    if shutil.which("g++") is None or _runtime("libasan.so") is None:
        pytest.skip("g++ with the AddressSanitizer runtime is not installed")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(CSRC, "attn_host.cpp"), os.path.join(CSRC, "rope_table.cpp"),
           os.path.join(HERE, "host_asan", "stubs.cpp"), "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    pre = _runtime("libasan.so")
    env["LD_PRELOAD"] = pre + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_asan", "run.py"), OUT], env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
