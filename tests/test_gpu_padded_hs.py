"""Head sizes 80 and 112 (block size b = 16) on the matrix-core kernel: the
kernels of head sizes 96 and 128 with the 16 missing columns zero in q' and
every code load kept inside the head's hs / 2 bytes (the lanes whose piece
would cross the row's end load it 8 bytes early). G1 (the written cache,
bit-exact) and G2 (atol = rtol = 1e-2 against the fp64 oracle on the cache the
GPU wrote) on every output row, for GQA and MHA decode, stream-K and split-KV,
multi-token decode and prefill tiles (one and two 16-row blocks), windows and
the inline-scale layout; the vector kernel meets the same gate on the same
inputs."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, host, kv4, oracle_attention_on_gpu_cache, oracle_caches, run_gpu

pytestmark = pytest.mark.gpu

G2 = dict(atol=1e-2, rtol=1e-2)

CASES = [
    # name, nq, nkv, query_lens, seq_lens, block_size
    ("decode_g4", 16, 4, [1] * 6, [4096, 17, 1000, 2049, 31, 700], 16),
    ("decode_g8_bs32", 32, 4, [1] * 3, [3000, 64, 513], 32),
    ("decode_mha", 8, 8, [1, 1], [900, 129], 16),
    ("decode_g2_nkv2", 4, 2, [1, 1, 1], [333, 16, 1500], 16),
    ("multi_token_g4", 16, 4, [3, 1, 4], [600, 40, 1500], 16),
    ("prefill_g2", 8, 4, [40, 1, 9], [300, 77, 9], 16),
    ("prefill_g6_two_blocks", 12, 2, [33, 5, 1], [400, 60, 1000], 16),
]


@pytest.mark.parametrize("path", ["auto", "valu"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("hs", [80, 112])
def test_padded_head_size_parity(hs, case, path, monkeypatch):
    if path == "valu":
        monkeypatch.setenv("KV4_FORCE_PATH", "valu")
    name, nq, nkv, ql, sl, bs = case
    r = run_gpu(W.custom(f"{name}_hs{hs}", nq, nkv, hs, ql, sl, block_size=bs, outlier_frac=0.01))
    okc, ovc, oks, ovs = oracle_caches(r)
    np.testing.assert_array_equal(host(r.kc), okc)
    np.testing.assert_array_equal(host(r.vc), ovc)
    ref = oracle_attention_on_gpu_cache(r)
    nbad, mx = allclose_report(host(r.out.float()), ref, **G2)
    assert nbad == 0, f"G2: {nbad} elements outside atol=rtol=1e-2 (max err {mx})"


@pytest.mark.parametrize("hs", [80, 112])
def test_padded_head_size_schedules(hs, monkeypatch):
    """Stream-K over a few workgroups (ranges straddling sequences) and small
    KV splits on the padded kernels: same gate."""
    w = W.custom(f"sched_hs{hs}", 16, 4, hs, [1] * 5, [2000, 33, 700, 1, 4096], block_size=16)
    for env in ({"KV4_SK_GRID": "3"}, {"KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "64"}):
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        r = run_gpu(w)
        ref = oracle_attention_on_gpu_cache(r)
        nbad, mx = allclose_report(host(r.out.float()), ref, **G2)
        assert nbad == 0, f"G2 {env}: {nbad} elements outside 1e-2 (max err {mx})"
        for k in env:
            monkeypatch.delenv(k)


@pytest.mark.parametrize("inline", [False, True], ids=["packed", "inline"])
@pytest.mark.parametrize("window", [0, 1, 100, 1000])
@pytest.mark.parametrize("hs", [80, 112])
def test_padded_head_size_layouts_and_windows(hs, window, inline):
    w = W.custom(f"win_hs{hs}", 16, 4, hs, [1, 5, 1, 40], [3000, 800, 40, 500], block_size=16)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb = lay.num_blocks
    if inline:
        cache = kv4.LayoutCache.inline("int4", nb, 16, 4, hs, device=DEV)
        kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, slots, sign_seed=w.sign_seed)
    else:
        kc = torch.zeros((nb, 16, 4, hs // 2), dtype=torch.uint8, device=DEV)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb, 16, 4), dtype=torch.float32, device=DEV)
        vs = torch.zeros_like(ks)
        kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, slots, sign_seed=w.sign_seed)
        cache = kv4.packed_layout_cache("int4", kc, vc, ks, vs)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed, sliding_window=window)
    torch.cuda.synchronize()
    if inline:
        kcn, vcn, ksn, vsn = O.inline_unpack(host(cache.buffer), "int4", 4, hs, 16)
    else:
        kcn, vcn, ksn, vsn = host(kc), host(vc), host(ks), host(vs)
    q = W.bf16_as_f32_numpy(t.query)
    ref = O.paged_attention(q, kcn, vcn, ksn, vsn, lay.block_table, lay.seq_lens, lay.query_start_loc,
                            hs ** -0.5, w.sign_seed, window=window)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    assert nbad == 0, f"G2 window {window}: {nbad} elements outside 1e-2 (max err {mx})"
