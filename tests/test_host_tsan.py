"""The library's host code (attn_host.cpp, rope_table.cpp) built with g++
under ThreadSanitizer against the thread-safe stand-in runtime of
host_tsan/stubs_tsan.cpp, and driven by host_tsan/tsan_driver.cpp: 16 threads
call every entry point at once, growing the RoPE tables while others read
them.  Any data race reported, or any unexpected status, fails the test.
CPU only."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "exact_scaled_dot_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_tsan")


def test_host_code_under_tsan():
    r = subprocess.run(["gcc", "-print-file-name=libtsan.so"], capture_output=True, text=True)
    if shutil.which("g++") is None or not os.path.isabs(r.stdout.strip()):
        pytest.skip("g++ with the ThreadSanitizer runtime is not installed")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-fPIE", "-pie",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(CSRC, "attn_host.cpp"), os.path.join(CSRC, "rope_table.cpp"),
           os.path.join(HERE, "host_tsan", "stubs_tsan.cpp"),
           os.path.join(HERE, "host_tsan", "tsan_driver.cpp"), "-o", OUT, "-lpthread"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    r = subprocess.run([OUT], env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-2000:]
    assert "unexpected statuses 0" in r.stdout, out[-2000:]
