"""The binding loads libattn.so into the HIP runtime torch uses: in a fresh
process that calls lib() before anything imports torch, and then imports
torch, exactly one HIP runtime library is mapped.  (torch ships its own runtime
and asks for it by another name than libattn.so does, so loading the library
first would leave two.)  CPU only: loading needs no GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import exact_scaled_dot_amd as esd
esd.lib()
import torch  # what a caller does next: the tensors come from torch
paths = set()
with open("/proc/self/maps") as f:
    for line in f:
        p = line.split()[-1]
        if "libamdhip64" in p:
            paths.add(p)
print(len(paths))
for p in sorted(paths):
    print(p)
"""


def test_one_hip_runtime_after_lib():
    import exact_scaled_dot_amd as esd
    if not os.path.exists(esd.LIB_PATH):
        pytest.skip("libattn.so is not built")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = r.stdout.split()
    assert lines[0] == "1", r.stdout
