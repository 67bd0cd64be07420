"""The -DKV4_DEBUG build (libkv4_debug.so, selected with KV4_LIBRARY in a
child process): valid calls raise no flag and give the release library's
output bits; a slot past the cache, a page id outside [0, num_blocks), a
seq_len beyond the page table and a decreasing query_start_loc each raise
their own KV4_DEBUG_* bit while the outputs stay finite (the kernels absorb
them)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import paged_decode_attention_reshape_amd as kv4
from paged_decode_attention_reshape_amd import build as B

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _child(lib, mode, *args, prefill="1"):
    env = dict(os.environ, KV4_LIBRARY=lib, KV4_PREFILL=prefill)
    r = subprocess.run([sys.executable, os.path.join(HERE, "debug_child.py"), mode, *args], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return [json.loads(ln) for ln in r.stdout.splitlines() if ln.startswith("{")]


def test_debug_build_valid_inputs_match_release(tmp_path):
    if not os.path.exists(B.DEBUG_LIB):
        pytest.skip("libkv4_debug.so is not built (__graft_entry__.build() builds it)")
    dbg = _child(B.DEBUG_LIB, "valid", str(tmp_path / "dbg.npz"))
    rel = _child(kv4.LIB_PATH, "valid", str(tmp_path / "rel.npz"))
    assert [r["flags"] for r in dbg] == [0, 0, 0], dbg
    assert [r["flags"] for r in rel] == [-1, -1, -1], rel   # the release library has no flags
    assert all(r["finite"] for r in dbg + rel)
    a, b = np.load(tmp_path / "dbg.npz"), np.load(tmp_path / "rel.npz")
    for k in a.files:
        np.testing.assert_array_equal(a[k], b[k])


def test_debug_build_flags_each_absorbed_input():
    if not os.path.exists(B.DEBUG_LIB):
        pytest.skip("libkv4_debug.so is not built (__graft_entry__.build() builds it)")
    res = {r["case"]: r for r in _child(B.DEBUG_LIB, "bad")}
    assert res["bad_slot"]["flags"] == kv4.KV4_DEBUG_SLOT
    assert res["bad_page"]["flags"] == kv4.KV4_DEBUG_PAGE
    assert res["bad_seqlen"]["flags"] == kv4.KV4_DEBUG_SEQLEN
    assert res["bad_qsl"]["flags"] & kv4.KV4_DEBUG_QSL
    assert all(r["finite"] for r in res.values())
