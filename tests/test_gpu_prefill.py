"""Chunked prefill on the prefill kernel (int4, head size 128): sequences with
more queries than four 32-row tiles hold (query_len > Q = 4 * (32 // group))
run on the workgroup-shared prefill kernel; beside it, single-query
sequences run as decode and those with 2 .. Q queries as query tiles in a
launch of their own (its partial rows per (query token, head) where the
batch has fewer tokens than sequences x Q, else per (sequence, query)), each
with its merge, in the same call. Every case checks G1 (the written cache, bit-exact)
and G2 (atol = rtol = 1e-2 against the fp64 oracle reading the cache the GPU
wrote) on every output row, with groups 1 to 32 (tiles of 32 // group
tokens), ragged last tiles, sequences of exactly one tile more than the
decode limit, long page tables, windows, the inline layout and rows with no
visible key."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, host, kv4, oracle_caches, run_gpu, say

pytestmark = pytest.mark.gpu

G2 = dict(atol=1e-2, rtol=1e-2)

CASES = [
    # name, nq, nkv, query_lens, seq_lens, block_size
    ("g1_mha", 4, 4, [33, 1, 64, 32], [33, 200, 1000, 40], 16),
    ("g2", 8, 4, [17, 100, 2, 16], [50, 700, 64, 300], 16),
    ("g3_ragged", 6, 2, [11, 45, 1, 10], [11, 300, 9, 1200], 16),
    ("g4_nkv8_streamk", 32, 8, [9, 129, 1, 8, 300], [9, 2000, 50, 130, 300], 16),
    ("g6_mixed", 12, 2, [6, 512, 1, 1, 21, 5], [2560, 1024, 8192, 17, 21, 5], 16),
    ("g8_bs32", 64, 8, [5, 77, 4], [100, 77, 4000], 32),
    ("g12_bs64", 24, 2, [3, 50, 2], [3, 900, 33], 64),
    ("g16_bs128", 32, 2, [3, 40, 2], [700, 40, 129], 128),
    ("g32", 32, 1, [2, 70, 1], [1000, 100, 65], 16),
    ("long_page_table", 12, 2, [600, 1], [5000, 3000], 16),
    ("only_prefill", 16, 4, [40, 41], [40, 3000], 16),
    # one chunk beside 127 three-query sequences: the 2 .. Q launch has more
    # units than its capped grid holds waves (grid-stride), token rows
    ("many_short_beside_chunk", 32, 8, [200] + [3] * 127,
     [1500] + [300 + (2700 * i) // 126 for i in range(127)], 16),
]


def _g1(r):
    okc, ovc, oks, ovs = oracle_caches(r)
    np.testing.assert_array_equal(host(r.kc), okc)
    np.testing.assert_array_equal(host(r.vc), ovc)
    np.testing.assert_array_equal(host(r.ks).view(np.uint32), oks.view(np.uint32))
    np.testing.assert_array_equal(host(r.vs).view(np.uint32), ovs.view(np.uint32))


def _g2_cache(w, lay, t, kc, vc, ks, vs, out, window=0):
    q = W.bf16_as_f32_numpy(t.query)
    ref = O.paged_attention(q, kc, vc, ks, vs, lay.block_table, lay.seq_lens, lay.query_start_loc,
                            w.head_size ** -0.5, w.sign_seed, window=window)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    say(f"    G2 max abs err {mx:.3e}, violations {nbad}")
    assert nbad == 0, f"G2: {nbad} elements outside atol=rtol=1e-2 (max err {mx})"
    return ref


@pytest.fixture(autouse=True)
def _prefill_on(monkeypatch):
    # the prefill kernel wherever the shape allows (by default it runs only
    # where long chunks carry the batch)
    monkeypatch.setenv("KV4_PREFILL", "1")


@pytest.mark.parametrize("prefill", ["on", "off", "auto"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(case, prefill, monkeypatch):
    """Every row of a mixed batch with the prefill kernel, without it (the
    single-kernel plan) and with the default choice: same gates."""
    if prefill == "off":
        monkeypatch.setenv("KV4_PREFILL", "0")
    if prefill == "auto":
        monkeypatch.delenv("KV4_PREFILL")
    name, nq, nkv, ql, sl, bs = case
    r = run_gpu(W.custom(name, nq, nkv, 128, ql, sl, block_size=bs))
    _g1(r)
    _g2_cache(r.w, r.lay, r.t, host(r.kc), host(r.vc), host(r.ks), host(r.vs), r.out)


def test_prefill_rows_before_the_context_are_zero():
    """Queries placed before the first cached key (query_len > seq_len) see no
    key: their rows are exactly 0, in prefill and decode sequences alike."""
    r = run_gpu(W.custom("q_gt_L", 12, 2, 128, [40, 20, 3], [30, 50, 1], block_size=16))
    ref = _g2_cache(r.w, r.lay, r.t, host(r.kc), host(r.vc), host(r.ks), host(r.vs), r.out)
    got = host(r.out.float())
    assert np.all(got[:10] == 0.0) and np.all(ref[:10] == 0.0)
    assert np.all(got[60:62] == 0.0)


WINDOWS = [1, 31, 64, 100, 1000]


@pytest.mark.parametrize("inline", [False, True], ids=["packed", "inline"])
@pytest.mark.parametrize("window", WINDOWS)
def test_prefill_sliding_window(window, inline):
    """Sliding windows on the prefill kernel (key ranges that start past the
    first 32-token step of the tile, and windows shorter than one step), on
    the packed and the inline (scales beside the codes, padded slots) layouts."""
    w = W.custom("pf_window", 12, 2, 128, [150, 1, 37, 6], [1200, 900, 300, 6], block_size=16)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb, bs, nkv, hs = lay.num_blocks, w.block_size, w.num_kv_heads, w.head_size
    if inline:
        cache = kv4.LayoutCache.inline("int4", nb, bs, nkv, hs, device=DEV)
        kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, slots, sign_seed=w.sign_seed)
    else:
        kc = torch.zeros((nb, bs, nkv, hs // 2), dtype=torch.uint8, device=DEV)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb, bs, nkv), dtype=torch.float32, device=DEV)
        vs = torch.zeros_like(ks)
        kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, slots, sign_seed=w.sign_seed)
        cache = kv4.packed_layout_cache("int4", kc, vc, ks, vs)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed, sliding_window=window)
    torch.cuda.synchronize()
    if inline:
        kcn, vcn, ksn, vsn = O.inline_unpack(host(cache.buffer), "int4", nkv, hs, bs)
    else:
        kcn, vcn, ksn, vsn = host(kc), host(vc), host(ks), host(vs)
    _g2_cache(w, lay, t, kcn, vcn, ksn, vsn, out, window=window)


def test_prefill_beyond_the_prefix_limit_runs_single_kernel():
    """More than 1024 sequences: the prefill kernel's in-kernel prefix does not
    cover them, and the call runs on the single-kernel plan (same gates)."""
    rng = np.random.default_rng(11)
    ql = [40 if i % 97 == 0 else 1 for i in range(1100)]
    sl = [int(x) + q for x, q in zip(rng.integers(1, 120, 1100), ql)]
    r = run_gpu(W.custom("many_seqs_prefill", 16, 4, 128, ql, sl, block_size=16))
    _g2_cache(r.w, r.lay, r.t, host(r.kc), host(r.vc), host(r.ks), host(r.vs), r.out)


def test_prefill_repeat_calls_are_bit_identical():
    """The prefill kernel has no order-dependent reduction across workgroups:
    the same call gives the same bits twice."""
    w = W.custom("pf_repeat", 12, 2, 128, [300, 1, 77], [2000, 500, 77], block_size=16)
    r = run_gpu(w)
    out2 = kv4.kv4_paged_attention(
        r.t.query.to(DEV), r.kc, r.vc, r.ks, r.vs, torch.from_numpy(r.lay.block_table).to(DEV),
        torch.from_numpy(r.lay.seq_lens).to(DEV), torch.from_numpy(r.lay.query_start_loc).to(DEV),
        max_query_len=w.max_query_len, max_seq_len=w.max_seq_len, sign_seed=w.sign_seed)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), r.out.view(torch.int16))


def test_prefill_side_stream_fork_matches_one_stream(monkeypatch):
    """With the prefill kernel, the decode kernel and the merge run on the
    library's side stream, forked from and joined back into the caller's
    stream: the bits equal those of the same kernels on one stream, also when
    the caller's stream is not the default one and the output is read on it
    right after the call."""
    w = W.custom("pf_fork", 12, 2, 128, [300, 1, 77, 1, 5], [2000, 500, 77, 3000, 64], block_size=16)
    r = run_gpu(w)
    args = (r.t.query.to(DEV), r.kc, r.vc, r.ks, r.vs, torch.from_numpy(r.lay.block_table).to(DEV),
            torch.from_numpy(r.lay.seq_lens).to(DEV), torch.from_numpy(r.lay.query_start_loc).to(DEV))
    kw = dict(max_query_len=w.max_query_len, max_seq_len=w.max_seq_len, sign_seed=w.sign_seed)
    monkeypatch.setenv("KV4_FORK", "0")
    one = kv4.kv4_paged_attention(*args, **kw)
    torch.cuda.synchronize()
    monkeypatch.setenv("KV4_FORK", "1")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            forked = kv4.kv4_paged_attention(*args, **kw, stream=s)
            copy = forked.clone()          # stream-ordered read right after the call
    s.synchronize()
    assert torch.equal(copy.view(torch.int16), one.view(torch.int16))
    assert torch.equal(r.out.view(torch.int16), one.view(torch.int16))
