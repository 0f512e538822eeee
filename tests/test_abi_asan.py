"""The C-ABI layer's host code under AddressSanitizer: the host-side ABI tests
(symbol exports, argument validation, workspace sizing, status strings) run
in a child process against libv4attn_asan.so, whose api.cpp is built with
-fsanitize=address, with the ASan runtime preloaded.  Any heap or stack
error in the host code aborts the child with an ASan report."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import pytest
from long_context_attention_v4attn_amd import binding
binding.load()
maps = open("/proc/self/maps").read()
assert "libv4attn_asan.so" in maps, "the ASan build is not the library loaded"
assert "libasan" in maps, "the ASan runtime is not loaded"
sys.exit(pytest.main(["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", "tests/test_abi.py"]))
"""


def test_abi_host_code_under_asan():
    from long_context_attention_v4attn_amd import build_asan
    try:
        lib = build_asan.build_asan()
        runtime = build_asan.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no host ASan toolchain: {e}")
    env = dict(os.environ, LD_PRELOAD=runtime, V4ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
