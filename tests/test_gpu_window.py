"""Sliding-window attention (kv4_attention_layout with sliding_window > 0):
G2 (atol = rtol = 1e-2) against the fp64 oracle with the same window, on the
cache the GPU wrote; decode (stream-K), mixed and prefill batches (split-KV),
both kernels, all three cache modes."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, host, kv4, say

pytestmark = pytest.mark.gpu

G2 = dict(atol=1e-2, rtol=1e-2)


def _run(w, mode, window, inline=False):
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb, bs, nkv, hs = lay.num_blocks, w.block_size, w.num_kv_heads, w.head_size
    if inline:
        cache = kv4.LayoutCache.inline(mode, nb, bs, nkv, hs, device=DEV)
        kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, slots, sign_seed=w.sign_seed)
    else:
        c = hs // 2 if mode == "int4" else hs
        kc = torch.zeros((nb, bs, nkv, c), dtype=torch.uint8, device=DEV)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb, bs, nkv), dtype=torch.float32, device=DEV)
        vs = torch.zeros_like(ks)
        if mode == "int4":
            kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, slots, sign_seed=w.sign_seed)
        else:
            kv4.kv4_pth_write(mode, t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, slots)
        cache = kv4.packed_layout_cache(mode, kc, vc, ks, vs)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed, sliding_window=window)
    torch.cuda.synchronize()
    if inline:
        kcn, vcn, ksn, vsn = O.inline_unpack(host(cache.buffer), mode, nkv, hs, bs)
    else:
        kcn, vcn, ksn, vsn = host(kc), host(vc), host(ks), host(vs)
    q = W.bf16_as_f32_numpy(t.query)
    if mode == "int4":
        ref = O.paged_attention(q, kcn, vcn, ksn, vsn, lay.block_table, lay.seq_lens, lay.query_start_loc,
                                hs ** -0.5, w.sign_seed, window=window)
    else:
        ref = O.pth_paged_attention(q, kcn, vcn, ksn, vsn, lay.block_table, lay.seq_lens, lay.query_start_loc,
                                    hs ** -0.5, mode, window=window)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    say(f"    {mode} window {window}: G2 max abs err {mx:.3e}, violations {nbad}")
    assert nbad == 0


CASES = [
    # name, nq, nkv, hs, query_lens, seq_lens, block_size
    ("decode_gqa4_hs128", 32, 8, 128, [1] * 5, [1000, 17, 300, 2049, 64], 16),
    ("decode_mha_hs96", 8, 8, 96, [1] * 3, [700, 40, 129], 16),
    ("mixed_prefill", 12, 2, 128, [1, 37, 1, 5, 1], [90, 300, 2000, 5, 64], 16),
    ("prefill_hs64_bs32", 8, 2, 64, [40, 3], [100, 77], 32),
    ("vector_path_bs8", 4, 2, 80, [1, 6], [333, 50], 8),
    ("multi_token_decode", 32, 8, 128, [3, 1, 4, 2], [700, 40, 1500, 5], 16),
]


@pytest.mark.parametrize("window", [1, 7, 32, 100, 1000])
@pytest.mark.parametrize("mode", ["int4", "int8", "fp8"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sliding_window(case, mode, window):
    name, nq, nkv, hs, ql, sl, bs = case
    say(f"[gpu] window {window} {mode} {name}")
    _run(W.custom(name, nq, nkv, hs, ql, sl, block_size=bs), mode, window)


SCHED = {
    "valu": {"KV4_FORCE_PATH": "valu"},
    "mfma_split64": {"KV4_FORCE_PATH": "mfma", "KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "64"},
    "mfma_split1000": {"KV4_FORCE_PATH": "mfma", "KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "1000"},
    "valu_split100": {"KV4_FORCE_PATH": "valu", "KV4_SPLIT_TOKENS": "100"},
    "streamk_grid3": {"KV4_SK_GRID": "3"},
    # the other merge form (one row per lane group) over windowed splits, and
    # the separate plan kernel with windowed stream-K steps
    "mfma_split64_merge_per_group": {"KV4_FORCE_PATH": "mfma", "KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "64",
                                     "KV4_REDUCE_ROWS": "1"},
    "streamk_plan_kernel": {"KV4_FUSED_PLAN": "0"},
    # one 16-row block per wave for the 9-token sequence (two by default)
    "mfma_one_row_block": {"KV4_FORCE_PATH": "mfma", "KV4_MFMA_RB": "1"},
}


@pytest.mark.parametrize("window", [5, 64, 250])
@pytest.mark.parametrize("sched", list(SCHED))
def test_sliding_window_schedules(sched, window, monkeypatch):
    for k, v in SCHED[sched].items():
        monkeypatch.setenv(k, v)
    _run(W.custom("sched", 16, 4, 128, [1, 1, 9, 1], [1500, 63, 700, 1], block_size=16), "int4", window)


@pytest.mark.parametrize("mode", ["int4", "fp8"])
def test_sliding_window_inline_layout(mode):
    _run(W.custom("inline", 32, 8, 128, [1] * 4, [900, 33, 2000, 128], block_size=16), mode, 200, inline=True)


def test_negative_window_rejected():
    w = W.custom("neg", 4, 4, 64, [1], [32], block_size=16)
    with pytest.raises(kv4.Kv4Error):
        _run(w, "int4", -1)
