"""Caller-described cache layouts on the GPU: the inline-scale padded-slot
layout and an arbitrary strided one, in all three modes.

Gates: the write is bit-exact over the whole buffer (codes and scales where
the oracle puts them, every other byte untouched); attention G2 (atol = rtol
= 1e-2) against the fp64 oracle reading the buffer the GPU wrote; dequant
against the oracle's float32 products.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, host, kv4, say

pytestmark = pytest.mark.gpu

MODES = ["int4", "int8", "fp8"]
G2 = dict(atol=1e-2, rtol=1e-2)


def _oracle_caches(mode, key, value, slots, nb, bs, seed):
    if mode == "int4":
        return O.write_kv(key, value, slots, nb, bs, seed)
    return O.pth_write_kv(key, value, slots, nb, bs, mode)


def _oracle_attention(mode, q, kc, vc, ks, vs, lay, scale, seed):
    if mode == "int4":
        return O.paged_attention(q, kc, vc, ks, vs, lay.block_table, lay.seq_lens, lay.query_start_loc, scale, seed)
    return O.pth_paged_attention(q, kc, vc, ks, vs, lay.block_table, lay.seq_lens, lay.query_start_loc, scale, mode)


def _inputs(w):
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = W.all_slots(lay, w)
    return lay, t, slots


CASES = [
    # name, nq, nkv, hs, query_lens, seq_lens, block_size
    ("gqa4_decode_hs128", 32, 8, 128, [1] * 4, [700, 17, 1500, 64], 16),
    ("mixed_hs96", 8, 2, 96, [1, 9, 1], [400, 40, 1000], 16),
    ("mha_hs64_bs32", 4, 4, 64, [1, 1, 2], [300, 33, 90], 32),
    ("hs192", 8, 2, 192, [1, 2], [500, 70], 16),
    ("hs80_bs8_vector_path", 4, 2, 80, [1, 3], [200, 31], 8),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_inline_layout_write_attention_dequant(case, mode):
    name, nq, nkv, hs, ql, sl, bs = case
    w = W.custom(name, nq, nkv, hs, ql, sl, block_size=bs, outlier_frac=0.02)
    say(f"[gpu] inline layout {mode} {name}")
    lay, t, slots = _inputs(w)
    nb = lay.num_blocks
    cache = kv4.LayoutCache.inline(mode, nb, bs, nkv, hs, device=DEV, fill=0xA5)
    kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, torch.from_numpy(slots).to(DEV),
                         sign_seed=w.sign_seed)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed)
    torch.cuda.synchronize()
    key, value, query = (W.bf16_as_f32_numpy(x) for x in (t.key, t.value, t.query))
    okc, ovc, oks, ovs = _oracle_caches(mode, key, value, slots, nb, bs, w.sign_seed)
    # write: whole buffer
    geo = O.inline_geometry(mode, nkv, hs, bs)
    want = np.full((nb, geo["block_bytes"]), 0xA5, dtype=np.uint8)
    O.inline_store_rows(want, okc, ovc, oks, ovs, slots, mode)
    got_buf = host(cache.buffer)
    nbad = int((got_buf != want).sum())
    assert nbad == 0, f"{nbad} buffer bytes differ"
    # attention on the GPU-written buffer
    kc, vc, ks, vs = O.inline_unpack(got_buf, mode, nkv, hs, bs)
    ref = _oracle_attention(mode, query, kc, vc, ks, vs, lay, hs ** -0.5, w.sign_seed)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    say(f"    G2 max abs err {mx:.3e}, violations {nbad}")
    assert nbad == 0
    # dequant of a few slots, incl. an out-of-range one
    q = slots[:64].copy()
    q[3] = -1
    d = host(kv4.kv4_dequant_layout(cache, "v", torch.from_numpy(q).to(DEV), sign_seed=w.sign_seed))
    qq = np.where(q < 0, 0, q)
    ref_d = O.dequant(vc, vs, qq, w.sign_seed, inverse_rotate=False) if mode == "int4" else O.pth_dequant(vc, vs, qq, mode)
    ref_d[3] = 0.0
    np.testing.assert_array_equal(d.view(np.uint32), ref_d.view(np.uint32))


SCHED = {
    "valu": {"KV4_FORCE_PATH": "valu"},
    "mfma_streamk": {"KV4_FORCE_PATH": "mfma"},
    "mfma_splits64": {"KV4_FORCE_PATH": "mfma", "KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "64"},
    # several kv heads per wave over rows whose heads are not adjacent (int4:
    # V staged per head; int8 / fp8 keep one head per wave)
    "mfma_hpw4": {"KV4_FORCE_PATH": "mfma", "KV4_MFMA_HPW": "4"},
    "mfma_hpw1": {"KV4_FORCE_PATH": "mfma", "KV4_MFMA_HPW": "1"},
}


@pytest.mark.parametrize("sched", list(SCHED))
@pytest.mark.parametrize("mode", MODES)
def test_inline_layout_paths_and_schedules(mode, sched, monkeypatch):
    for k, v in SCHED[sched].items():
        monkeypatch.setenv(k, v)
    w = W.custom("sched", 16, 4, 128, [1] * 5, [900, 5, 333, 2049, 64], block_size=16)
    lay, t, slots = _inputs(w)
    cache = kv4.LayoutCache.inline(mode, lay.num_blocks, 16, 4, 128, device=DEV)
    kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, torch.from_numpy(slots).to(DEV),
                         sign_seed=w.sign_seed)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed)
    torch.cuda.synchronize()
    kc, vc, ks, vs = O.inline_unpack(host(cache.buffer), mode, 4, 128, 16)
    ref = _oracle_attention(mode, W.bf16_as_f32_numpy(t.query), kc, vc, ks, vs, lay, 128 ** -0.5, w.sign_seed)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    assert nbad == 0, f"G2 violations {nbad} (max err {mx})"


@pytest.mark.parametrize("mode", MODES)
def test_head_major_layout_with_separate_scale_order(mode):
    """Codes [nb, nkv, bs, C] (head-major pages) and scales [nkv, nb, bs]:
    strides unlike any packed layout."""
    nq, nkv, hs, bs = 8, 2, 128, 16
    w = W.custom("headmajor", nq, nkv, hs, [1, 4, 1], [600, 50, 129], block_size=bs)
    lay, t, slots = _inputs(w)
    nb = lay.num_blocks
    c = hs // 2 if mode == "int4" else hs
    kbuf = torch.full((nb, nkv, bs, c), 0x5A, dtype=torch.uint8, device=DEV)
    vbuf = torch.full_like(kbuf, 0x5A)
    ksb = torch.zeros((nkv, nb, bs), dtype=torch.float32, device=DEV)
    vsb = torch.zeros_like(ksb)
    L = kv4.CacheLayout(nkv * bs * c, c, bs * c, bs, 1, nb * bs)
    cache = kv4.LayoutCache(mode, L, nb, bs, nkv, hs, kbuf.data_ptr(), vbuf.data_ptr(), ksb.data_ptr(),
                            vsb.data_ptr(), (kbuf, vbuf, ksb, vsb))
    kv4.kv4_write_layout(t.key.to(DEV), t.value.to(DEV), cache, torch.from_numpy(slots).to(DEV),
                         sign_seed=w.sign_seed)
    out = kv4.kv4_attention_layout(t.query.to(DEV), cache, torch.from_numpy(lay.block_table).to(DEV),
                                   torch.from_numpy(lay.seq_lens).to(DEV),
                                   torch.from_numpy(lay.query_start_loc).to(DEV), w.max_query_len, w.max_seq_len,
                                   sign_seed=w.sign_seed)
    torch.cuda.synchronize()
    key, value, query = (W.bf16_as_f32_numpy(x) for x in (t.key, t.value, t.query))
    okc, ovc, oks, ovs = _oracle_caches(mode, key, value, slots, nb, bs, w.sign_seed)
    # back to the packed order: codes [nb, bs, nkv, c], scales [nb, bs, nkv]
    kc = host(kbuf).transpose(0, 2, 1, 3)
    vc = host(vbuf).transpose(0, 2, 1, 3)
    ks = host(ksb).transpose(1, 2, 0)
    vs = host(vsb).transpose(1, 2, 0)
    written = np.zeros((nb * bs,), dtype=bool)
    written[slots] = True
    wr = written.reshape(nb, bs)
    np.testing.assert_array_equal(kc[wr], okc[wr])
    np.testing.assert_array_equal(vc[wr], ovc[wr])
    np.testing.assert_array_equal(ks[wr].view(np.uint32), oks[wr].view(np.uint32))
    np.testing.assert_array_equal(vs[wr].view(np.uint32), ovs[wr].view(np.uint32))
    assert (kc[~wr] == 0x5A).all() and (vc[~wr] == 0x5A).all()
    ref = _oracle_attention(mode, query, np.ascontiguousarray(kc), np.ascontiguousarray(vc),
                            np.ascontiguousarray(ks), np.ascontiguousarray(vs), lay, hs ** -0.5, w.sign_seed)
    nbad, mx = allclose_report(host(out.float()), ref, **G2)
    assert nbad == 0, f"G2 violations {nbad} (max err {mx})"
