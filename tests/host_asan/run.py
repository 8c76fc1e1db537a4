"""Run the host-side ABI tests against the sanitizer build of the library's
host code (argument: path of that library).  Started by test_host_sanitized.py
in a process that has the AddressSanitizer runtime preloaded; test
infrastructure only."""

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
sys.path[:0] = [ROOT, TESTS]

import exact_scaled_dot_amd as esd  # noqa: E402
import pytest  # noqa: E402


def main(path):
    L = esd._declare(ctypes.CDLL(path))
    esd._lib = L  # the binding's lib() now returns the sanitizer build
    os.environ["ATTN_SAN_LIB"] = path
    # -s: a sanitizer report goes straight to stderr (the run stops at the first)
    return pytest.main(["-q", "-s", "-p", "no:cacheprovider", "-o", "addopts=",
                        os.path.join(TESTS, "test_abi.py"), os.path.join(HERE, "check_dispatch.py"),
                        os.path.join(HERE, "fuzz_args.py")])


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
