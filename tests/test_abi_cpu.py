"""C-ABI checks that need no GPU: the library loads, exports every function
include/kv4.h declares, and rejects invalid arguments on the host before any
HIP call (no kernel is launched by anything here)."""
import ctypes
import os
import subprocess

import pytest

import paged_decode_attention_reshape_amd as kv4
from paged_decode_attention_reshape_amd.build import build_library

EINVAL, EWORKSPACE, EUNSUPPORTED = kv4.KV4_EINVAL, kv4.KV4_EWORKSPACE, kv4.KV4_EUNSUPPORTED


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kv4.LIB_PATH):
        build_library()
    return kv4.lib()


def test_header_declares_the_boundary():
    assert kv4.header_functions() == sorted([
        "kv4_dequant", "kv4_last_error", "kv4_paged_attention",
        "kv4_paged_attention_workspace_size", "kv4_rht_write",
        "kv4_pth_write", "kv4_pth_dequant", "kv4_pth_attention", "kv4_pth_attention_workspace_size",
        "kv4_cache_layout_packed", "kv4_cache_layout_inline", "kv4_write_layout",
        "kv4_attention_layout_workspace_size", "kv4_attention_layout", "kv4_dequant_layout",
        "kv4_stream_read", "kv4_paged_attention_noalloc", "kv4_debug_flags"])


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", kv4.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in kv4.header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_binding_names_match_c_names():
    for name in kv4.header_functions():
        assert callable(getattr(kv4, name)), name


def _write(L, **over):
    args = dict(key=16, value=16, ks=192, vs=192, kc=16, vc=16, ksc=16, vsc=16, slots=16, T=4, nkv=2, hs=96,
                b=32, bs=16, nb=4, seed=42)
    args.update(over)
    a = args
    return L.kv4_rht_write(a["key"], a["value"], a["ks"], a["vs"], a["kc"], a["vc"], a["ksc"], a["vsc"],
                           a["slots"], a["T"], a["nkv"], a["hs"], a["b"], a["bs"], a["nb"], a["seed"], None)


@pytest.mark.parametrize("over,needle", [
    (dict(hs=100, b=4), "multiple of 8"),
    (dict(hs=264, b=8), "multiple of 8"),
    (dict(hs=96, b=96), "largest power of two"),
    (dict(hs=96, b=16), "largest power of two"),
    (dict(hs=128, b=64), "largest power of two"),
    (dict(nkv=0), "num_kv_heads"),
    (dict(bs=0), "block_size"),
    (dict(T=-1), "num_tokens"),
    (dict(ks=100), "stride"),
    (dict(ks=194), "stride"),
    (dict(key=0), "null"),
    (dict(slots=0), "null"),
    (dict(kc=8), "misaligned"),
    (dict(key=24), "misaligned"),
])
def test_write_validation(L, over, needle):
    assert _write(L, **over) == EINVAL
    assert needle in kv4.kv4_last_error()


def test_write_accepts_non_power_of_two_heads_noop(L):
    """Every head size that is a multiple of 8 is accepted (the pages' abort
    on head_size 96 is the failure this guards against); num_tokens == 0 is a
    valid no-op that launches nothing."""
    for hs in range(8, 257, 8):
        assert _write(L, hs=hs, b=hs & -hs, ks=2 * hs, vs=2 * hs, T=0) == 0, kv4.kv4_last_error()
    assert kv4.kv4_last_error() == ""


def test_b_zero_derives_the_rule(L):
    """b = 0 asks the library for the largest power of two dividing head_size:
    accepted for every head size (checked before the no-op return), while a
    wrong nonzero b is still rejected."""
    for hs in range(8, 257, 8):
        assert _write(L, hs=hs, b=0, ks=2 * hs, vs=2 * hs, T=0) == 0, kv4.kv4_last_error()
        assert L.kv4_dequant(16, 16, 4, 16, 0, 2, hs, 0, 16, 42, 1, 16, None) == 0, kv4.kv4_last_error()
    assert _write(L, hs=96, b=96, T=0) == EINVAL
    assert _attn(L, b=0, Tq=0, S=0) == 0, kv4.kv4_last_error()
    assert _attn(L, b=0, hs=100, Tq=0, S=0) == EINVAL


def test_entry_points_return_kv4_status():
    """The header declares every work entry point as returning kv4_status."""
    import re
    text = re.sub(r"/\*.*?\*/", "", open(kv4.HEADER_PATH).read(), flags=re.S)
    for name in kv4.header_functions():
        m = re.search(r"^([A-Za-z_0-9 ]+\**)\s*" + name + r"\(", text, flags=re.M)
        assert m, name
        want = {"kv4_last_error": "const char*"}.get(name, "size_t" if name.endswith("workspace_size")
                                                    else "kv4_status")
        assert m.group(1).strip() == want, (name, m.group(1))


def _attn(L, **over):
    a = dict(q=16, qs=8 * 96, kc=16, vc=16, ksc=16, vsc=16, nb=10, bt=16, maxb=4, sl=16, qsl=16, S=2, Tq=2,
             mql=1, msl=64, nq=8, nkv=2, hs=96, b=32, bs=16, seed=42, scale=0.1, out=16, ws=0, wsb=0)
    a.update(over)
    return L.kv4_paged_attention(a["q"], a["qs"], a["kc"], a["vc"], a["ksc"], a["vsc"], a["nb"], a["bt"],
                                 a["maxb"], a["sl"], a["qsl"], a["S"], a["Tq"], a["mql"], a["msl"], a["nq"],
                                 a["nkv"], a["hs"], a["b"], a["bs"], a["seed"], a["scale"], a["out"], a["ws"],
                                 a["wsb"], None)


@pytest.mark.parametrize("over,needle", [
    (dict(hs=97), "multiple of 8"),
    (dict(b=96), "largest power of two"),
    (dict(nq=7), "multiple of num_kv_heads"),
    (dict(nkv=0), "num_kv_heads"),
    (dict(S=0), "num_seqs"),
    (dict(Tq=-3), "num_q_tokens"),
    (dict(maxb=0), "max_blocks_per_seq"),
    (dict(qs=8), "query_token_stride"),
    (dict(scale=float("inf")), "softmax_scale"),
    (dict(q=0), "null"),
    (dict(out=8), "misaligned"),
    (dict(mql=-1), "max lengths"),
])
def test_attention_validation(L, over, needle):
    assert _attn(L, **over) == EINVAL
    assert needle in kv4.kv4_last_error()


def test_attention_rejects_2_31_query_rows(L):
    # the merge numbers (query token, query head) rows in 32 bits
    assert _attn(L, Tq=1 << 28, nq=8, qs=8 * 96, qsl=16, mql=1) == kv4.KV4_EUNSUPPORTED
    assert "2^31" in kv4.kv4_last_error()


def test_attention_workspace_required(L):
    need = L.kv4_paged_attention_workspace_size(2, 2, 8, 2, 96, 1, 100000)
    assert need > 0
    assert _attn(L, msl=100000, ws=0, wsb=0) == EWORKSPACE
    assert "workspace" in kv4.kv4_last_error()
    assert _attn(L, msl=100000, ws=256, wsb=need - 1) == EWORKSPACE


def test_workspace_size(L):
    # no query tokens -> no workspace; single-token decode on the matrix cores
    # (stream-K) -> the per-sequence prefix plus at most (2048 workgroups +
    # num_seqs) pieces of hs + 2 floats per query head
    assert L.kv4_paged_attention_workspace_size(0, 0, 8, 2, 96, 0, 0) == 0
    short = L.kv4_paged_attention_workspace_size(4096, 4096, 8, 8, 128, 1, 200)
    bound = (4 * 4097 + 255) // 256 * 256 + (2048 + 4096) * 8 * (128 + 2) * 4 + 2 * 256
    assert 0 < short <= bound
    # long contexts are split: partial rows of hs + 2 floats per split
    n = L.kv4_paged_attention_workspace_size(128, 128, 32, 8, 128, 1, 32768)
    assert n >= 2 * 128 * 32 * 130 * 4
    # invalid sizes give 0 and a message
    assert L.kv4_paged_attention_workspace_size(4, 1, 7, 2, 96, 1, 10) == 0
    assert "multiple" in kv4.kv4_last_error()


def test_prefill_plan_compacts_the_split_rows(L, monkeypatch):
    # A chunked-prefill batch (Qwen2.5-1.5B shape: 12/2 heads, hs 128, 4 x 512
    # prefill + 60 decode tokens): the prefill sequences run on the prefill
    # kernel, so the split partial rows are only those of the single-query
    # sequences -- (split, sequence) rows instead of (split, query token) rows
    # over all 2108 tokens.
    monkeypatch.setenv("KV4_PREFILL", "1")
    args = (2108, 64, 12, 2, 128, 512, 8192)
    with_pf = L.kv4_paged_attention_workspace_size(*args)
    monkeypatch.setenv("KV4_PREFILL", "0")
    without = L.kv4_paged_attention_workspace_size(*args)
    assert 0 < with_pf < without
    # the same plan with more sequences than the prefill kernel's prefix holds
    # (1100 > 1024) falls back to the single-kernel layout
    monkeypatch.setenv("KV4_PREFILL", "1")
    many = (1100 + 4 * 512, 1104, 12, 2, 128, 512, 8192)
    a = L.kv4_paged_attention_workspace_size(*many)
    monkeypatch.setenv("KV4_PREFILL", "0")
    assert a == L.kv4_paged_attention_workspace_size(*many)
    # by default the prefill kernel runs where a sequence may have more than
    # Q = 4 tiles of queries (20 at group 6) and the tokens beyond one per
    # sequence could fill 128 of its workgroups ((T - S) x kv heads >= 128 Q):
    # the 4 x 512 chunks with or without the 60 decode sequences, not 4 x 64
    # chunks among them (504 < 2560) nor short multi-query sequences alone
    monkeypatch.delenv("KV4_PREFILL")
    assert L.kv4_paged_attention_workspace_size(*args) == with_pf
    only = (2048, 4, 12, 2, 128, 512, 2560)
    auto = L.kv4_paged_attention_workspace_size(*only)
    small = (4 * 64 + 60, 64, 12, 2, 128, 64, 8192)
    short = (415, 64, 12, 2, 128, 12, 8192)
    auto_small = L.kv4_paged_attention_workspace_size(*small)
    auto_short = L.kv4_paged_attention_workspace_size(*short)
    monkeypatch.setenv("KV4_PREFILL", "0")
    assert auto < L.kv4_paged_attention_workspace_size(*only)
    assert auto_small == L.kv4_paged_attention_workspace_size(*small)
    assert auto_short == L.kv4_paged_attention_workspace_size(*short)
    monkeypatch.setenv("KV4_PREFILL", "1")
    assert L.kv4_paged_attention_workspace_size(*small) != auto_small


@pytest.mark.parametrize("shape", [
    # (T, S, nq, nkv, max_query_len, max_seq_len): one chunk beside 64
    # four-query sequences (Llama-3-8B shape); the mixed Qwen2.5-1.5B batch;
    # 4 chunks of 512 beside 60 four-query sequences and 4 decodes (Qwen shape)
    (768, 65, 32, 8, 512, 32768),
    (2108, 64, 12, 2, 512, 8192),
    (4 * 512 + 60 * 4 + 4, 68, 12, 2, 512, 8192),
])
def test_prefill_plan_multi_query_launch_stays_within_the_single_kernel_plan(L, monkeypatch, shape):
    # Beside the prefill kernel the launch of the 2 .. Q-query sequences
    # splits no finer than the single-kernel plan and has at most as many
    # partial rows per split, so the call's workspace exceeds that plan's by
    # at most the single-query launch's (its per-sequence prefix and at most
    # 2048 + S stream-K pieces, or S rows per split of at least 512 tokens)
    T, S, nq, nkv, mq, msl = shape
    monkeypatch.setenv("KV4_PREFILL", "0")
    single = L.kv4_paged_attention_workspace_size(T, S, nq, nkv, 128, mq, msl)
    monkeypatch.setenv("KV4_PREFILL", "1")
    with_pf = L.kv4_paged_attention_workspace_size(T, S, nq, nkv, 128, mq, msl)
    row = nq * (128 + 2) * 4
    decode = max((2048 + S) * row, S * row * -(-msl // 512)) + 3 * (4 * (S + 1) + 256) + 4 * 256
    assert 0 < single and 0 < with_pf <= single + decode


def test_dequant_validation(L):
    rc = L.kv4_dequant(16, 16, 4, 16, 3, 2, 96, 64, 16, 42, 1, 16, None)
    assert rc == EINVAL and "largest power of two" in kv4.kv4_last_error()
    rc = L.kv4_dequant(16, 16, 4, 16, 0, 2, 96, 32, 16, 42, 1, 16, None)
    assert rc == 0
    rc = L.kv4_dequant(0, 16, 4, 16, 3, 2, 96, 32, 16, 42, 1, 16, None)
    assert rc == EINVAL and "null" in kv4.kv4_last_error()


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((2, 2, 96), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kv4.kv4_rht_write(x, x, torch.zeros((1, 16, 2, 48), dtype=torch.uint8),
                          torch.zeros((1, 16, 2, 48), dtype=torch.uint8),
                          torch.zeros((1, 16, 2)), torch.zeros((1, 16, 2)), torch.zeros(2, dtype=torch.int64))


def test_pth_mode_validation(L):
    # kv_quant_mode must be 1 (int8) or 2 (fp8); checked before anything else
    rc = L.kv4_pth_write(3, 16, 16, 64, 64, 16, 16, 16, 16, 16, 4, 1, 64, 16, 4, None)
    assert rc == EINVAL and "kv_quant_mode" in kv4.kv4_last_error()
    rc = L.kv4_pth_write(1, 16, 16, 64, 64, 16, 16, 16, 16, 16, 4, 1, 60, 16, 4, None)
    assert rc == EINVAL and "multiple of 8" in kv4.kv4_last_error()
    rc = L.kv4_pth_dequant(2, 16, 16, 4, 16, 0, 1, 64, 16, 16, None)
    assert rc == 0
    rc = L.kv4_pth_dequant(0, 16, 16, 4, 16, 3, 1, 64, 16, 16, None)
    assert rc == EINVAL
    with pytest.raises(ValueError):
        kv4._mode("int4")


def test_cache_layouts_on_the_host():
    """Packed and inline layouts (host-only helpers; no GPU needed)."""
    p = kv4.kv4_cache_layout_packed("int4", 8, 128, 16).as_tuple()
    assert p == (16 * 8 * 64, 8 * 64, 64, 16 * 8, 8, 1)
    p = kv4.kv4_cache_layout_packed("fp8", 2, 96, 32).as_tuple()
    assert p == (32 * 2 * 96, 2 * 96, 96, 32 * 2, 2, 1)
    lay, bb, vo, so = kv4.kv4_cache_layout_inline("int4", 8, 128, 16)
    # 64 code bytes + 4-byte scale -> 80-byte rows; K half then V half
    assert (bb, vo, so) == (2 * 16 * 8 * 80, 16 * 8 * 80, 64)
    assert lay.as_tuple() == (bb, 8 * 80, 80, bb // 4, 8 * 80 // 4, 80 // 4)
    lay, bb, vo, so = kv4.kv4_cache_layout_inline("int8", 3, 8, 1)
    assert (lay.head_stride, so, bb) == (16, 8, 2 * 3 * 16)
    with pytest.raises(kv4.Kv4Error):
        kv4.kv4_cache_layout_inline("int4", 0, 128, 16)
    with pytest.raises(ValueError):
        kv4.kv4_cache_layout_inline("int2", 8, 128, 16)


def test_invalid_layouts_are_rejected_on_the_host():
    good = kv4.kv4_cache_layout_inline("int8", 2, 64, 16)[0]

    class C:   # a LayoutCache stand-in; only its sizes and layout are read
        mode, num_kv_heads, head_size = 1, 2, 64

    def ws(t):
        c = C()
        c.layout = kv4.CacheLayout(*t)
        return kv4.kv4_attention_layout_workspace_size(c, 4, 2, 8, 1, 100)

    assert ws(good.as_tuple()) >= 0
    for bad in [(0, 128, 64, 10, 5, 1),            # zero stride
                (4096, 132, 64, 10, 5, 1),         # int8 code stride not a multiple of 8
                (4096, 128, 64, 10, 5, -1)]:       # negative scale stride
        with pytest.raises(kv4.Kv4Error):
            ws(bad)


def test_planner_sweep_workspace_sizes(L):
    """The host planner and workspace layout over a grid of shapes (head
    sizes, groups, query and sequence lengths, batch sizes, all three cache
    modes, packed and inline layouts): every valid shape is planned without
    an error (a single-split plan on the vector kernel needs no workspace at
    all), a plan on the matrix cores needs some (the sequence prefix), and
    no query tokens need none."""
    import itertools
    for hs, (nq, nkv), mql, msl, S, qm in itertools.product(
            (8, 64, 96, 128, 192, 256), ((8, 8), (32, 8), (12, 2), (64, 1)), (1, 5, 600), (1, 100, 70000),
            (1, 7, 1500), (0, 1, 2)):
        Tq = S * mql
        if qm == 0:
            n = L.kv4_paged_attention_workspace_size(Tq, S, nq, nkv, hs, mql, msl)
        else:
            n = L.kv4_pth_attention_workspace_size(qm, Tq, S, nq, nkv, hs, mql, msl)
        assert kv4.kv4_last_error() == "", (hs, nq, nkv, mql, msl, S, qm, kv4.kv4_last_error())
        assert n % 256 == 0
        if hs in (64, 96, 128, 192):           # matrix-core plans keep the sequence prefix there
            assert n > 0, (hs, nq, nkv, mql, msl, S, qm)
        lay, bb, vo, so = kv4.kv4_cache_layout_inline(qm, nkv, hs, 16)
        L.kv4_attention_layout_workspace_size(qm, ctypes.byref(lay), Tq, S, nq, nkv, hs, mql, msl)
        assert kv4.kv4_last_error() == ""
        assert L.kv4_paged_attention_workspace_size(0, S, nq, nkv, hs, mql, msl) == 0


def test_debug_flags_need_a_debug_build(L):
    import ctypes
    v = ctypes.c_uint32(7)
    assert L.kv4_debug_flags(ctypes.byref(v), 0) == EUNSUPPORTED
    assert v.value == 0 and "KV4_DEBUG" in kv4.kv4_last_error()
    assert L.kv4_debug_flags(None, 0) == EINVAL


def test_debug_library_exports_the_same_abi():
    """libkv4_debug.so (built with -DKV4_DEBUG) exports every symbol of the
    header, like the release library."""
    import os
    import subprocess
    from paged_decode_attention_reshape_amd import build as B
    if not os.path.exists(B.DEBUG_LIB):
        B.build_debug_library()
    out = subprocess.run(["nm", "-D", "--defined-only", B.DEBUG_LIB], capture_output=True, text=True,
                         check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [f for f in kv4.header_functions() if f not in names]
    assert not missing, missing
