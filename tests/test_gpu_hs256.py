"""Head size 256 on the matrix-core kernel (one kv head per wave, one wave per
SIMD): G1 (bit-exact cache) and G2 (atol = rtol = 1e-2 against the fp64
oracle on the cache the GPU wrote) for GQA decode, multi-token decode,
prefill chunks, sliding windows and the int8 / fp8 caches, on every output
row; the vector kernel on the same inputs meets the same gate."""
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
    ("multi_token_g4", 16, 4, [3, 1, 4], [600, 40, 1500], 16),
    ("prefill_g2", 8, 4, [40, 1, 9], [300, 77, 9], 16),
]


@pytest.mark.parametrize("path", ["auto", "valu"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hs256_parity(case, path, monkeypatch):
    if path == "valu":
        monkeypatch.setenv("KV4_FORCE_PATH", "valu")
    name, nq, nkv, ql, sl, bs = case
    r = run_gpu(W.custom(name, nq, nkv, 256, ql, sl, block_size=bs, outlier_frac=0.01))
    okc, ovc, oks, ovs = oracle_caches(r)
    np.testing.assert_array_equal(host(r.kc), okc)
    np.testing.assert_array_equal(host(r.vc), ovc)
    ref = oracle_attention_on_gpu_cache(r)
    nbad, mx = allclose_report(host(r.out.float()), ref, **G2)
    assert nbad == 0, f"G2: {nbad} elements outside atol=rtol=1e-2 (max err {mx})"


@pytest.mark.parametrize("mode", ["int8", "fp8"])
def test_hs256_per_token_head_caches(mode):
    w = W.custom("pth256", 16, 4, 256, [1, 2, 1], [2000, 300, 64], block_size=16)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb = lay.num_blocks
    kc = torch.zeros((nb, 16, 4, 256), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((nb, 16, 4), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    kv4.kv4_pth_write(mode, t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, slots)
    out = kv4.kv4_pth_attention(mode, t.query.to(DEV), kc, vc, ks, vs, torch.from_numpy(lay.block_table).to(DEV),
                                torch.from_numpy(lay.seq_lens).to(DEV), torch.from_numpy(lay.query_start_loc).to(DEV),
                                w.max_query_len, w.max_seq_len)
    torch.cuda.synchronize()
    q = W.bf16_as_f32_numpy(t.query)
    ref = O.pth_paged_attention(q, host(kc), host(vc), host(ks), host(vs), lay.block_table, lay.seq_lens,
                                lay.query_start_loc, 256 ** -0.5, mode)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    assert nbad == 0, f"G2 {mode}: {nbad} elements outside 1e-2 (max err {mx})"


@pytest.mark.parametrize("window", [1, 100, 1000])
def test_hs256_window(window):
    w = W.custom("win256", 16, 4, 256, [1, 5, 1], [3000, 800, 40], block_size=16)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb = lay.num_blocks
    kc = torch.zeros((nb, 16, 4, 128), dtype=torch.uint8, device=DEV)
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
    q = W.bf16_as_f32_numpy(t.query)
    ref = O.paged_attention(q, host(kc), host(vc), host(ks), host(vs), lay.block_table, lay.seq_lens,
                            lay.query_start_loc, 256 ** -0.5, w.sign_seed, window=window)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    assert nbad == 0, f"G2 window {window}: {nbad} elements outside 1e-2 (max err {mx})"
