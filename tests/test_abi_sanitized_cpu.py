"""The C ABI's host code (argument validation, the launch planner, the
workspace layout) under AddressSanitizer and UndefinedBehaviorSanitizer: a
build of libkv4 whose kv4_api.cpp is instrumented on the host, loaded with the
clang ASan runtime preloaded, runs the ABI tests of test_abi_cpu.py in a child
process. Any out-of-bounds access, use after free, signed overflow or other
undefined behaviour there aborts the child. No GPU is needed (nothing here
launches a kernel)."""
import os
import subprocess
import sys

import pytest

from paged_decode_attention_reshape_amd.build import asan_runtime, build_sanitized_library

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import paged_decode_attention_reshape_amd as kv4
kv4.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {tests!r} + '/test_abi_cpu.py'])
assert kv4.lib()._name == {lib!r}
sys.exit(int(rc))
"""


def test_abi_under_asan_and_ubsan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    lib = build_sanitized_library()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=HERE, lib=lib)], env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
