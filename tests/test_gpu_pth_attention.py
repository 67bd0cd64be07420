"""Read path parity of the per-token-head INT8 / FP8 control modes.

Gates (tolerances are written here, in the tests):
  G1  the caches kv4_pth_write fills are bit-exact against the oracle's.
  G2  kv4_pth_attention vs the fp64 oracle reading the cache the GPU wrote:
      atol = rtol = 1e-2.
  G4  vs unquantized fp64 attention: int8 within atol = rtol = 5e-2; fp8 (3
      mantissa bits) reports its error and must keep correlation > 0.99.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, corr, host, kv4, say

pytestmark = pytest.mark.gpu

MODES = ["int8", "fp8"]
G2 = dict(atol=1e-2, rtol=1e-2)
G4 = dict(atol=5e-2, rtol=5e-2)


def _run(w, mode, softmax_scale=None, q_gain=1.0):
    say(f"[gpu] pth attention {mode} case {w.name}: nq={w.num_q_heads} nkv={w.num_kv_heads} "
        f"hs={w.head_size} bs={w.block_size} seqs={w.num_seqs} q_tokens={w.num_q_tokens}")
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = W.all_slots(lay, w)
    nkv, hs, bs = w.num_kv_heads, w.head_size, w.block_size
    kc = torch.zeros((lay.num_blocks, bs, nkv, hs), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((lay.num_blocks, bs, nkv), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    if q_gain != 1.0:
        t.query = (t.query.float() * q_gain).to(torch.bfloat16)
    kv4.kv4_pth_write(mode, t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, torch.from_numpy(slots).to(DEV))
    out = kv4.kv4_pth_attention(
        mode, t.query.to(DEV), kc, vc, ks, vs, torch.from_numpy(lay.block_table).to(DEV),
        torch.from_numpy(lay.seq_lens).to(DEV), torch.from_numpy(lay.query_start_loc).to(DEV),
        max_query_len=w.max_query_len, max_seq_len=w.max_seq_len, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    key, value, query = (W.bf16_as_f32_numpy(x) for x in (t.key, t.value, t.query))
    # G1
    okc, ovc, oks, ovs = O.pth_write_kv(key, value, slots, lay.num_blocks, bs, mode)
    np.testing.assert_array_equal(host(kc), okc)
    np.testing.assert_array_equal(host(vc), ovc)
    np.testing.assert_array_equal(host(ks).view(np.uint32), oks.view(np.uint32))
    np.testing.assert_array_equal(host(vs).view(np.uint32), ovs.view(np.uint32))
    # G2
    sc = hs ** -0.5 if softmax_scale is None else softmax_scale
    ref = O.pth_paged_attention(query, host(kc), host(vc), host(ks), host(vs), lay.block_table, lay.seq_lens,
                                lay.query_start_loc, sc, mode)
    got = host(out.float())
    live = ~np.isnan(ref)
    nbad, mx = allclose_report(got[live], ref[live], **G2)
    say(f"    G2 max abs err {mx:.3e}, violations {nbad}")
    assert nbad == 0, f"G2: {nbad} elements outside atol=rtol=1e-2 (max err {mx})"
    return lay, key, value, query, got, ref, sc


CASES = [
    # name, nq, nkv, hs, query_lens, seq_lens, block_size
    ("tiny_L32", 4, 4, 128, [1], [32], 16),
    ("partial_page_q4", 4, 4, 128, [4, 4], [128, 97], 16),
    ("phi3_like_hs96", 8, 8, 96, [1] * 5, [1024, 17, 300, 33, 512], 16),
    ("gqa4_hs64", 8, 2, 64, [1] * 6, [1000, 1, 16, 17, 2049, 160], 16),
    ("gqa6_hs128_mixed", 12, 2, 128, [1, 37, 1, 5, 1], [90, 300, 2000, 5, 64], 16),
    ("hs192", 8, 2, 192, [1, 3], [700, 129], 16),
    ("hs192_mha_odd_heads", 6, 6, 192, [1, 1], [333, 1030], 16),
    ("hs96_prefill", 8, 4, 96, [17, 1], [40, 500], 32),
    ("hs80", 4, 1, 80, [1, 2], [333, 50], 16),
    ("hs256", 4, 2, 256, [1, 1], [100, 257], 16),
    ("hs8", 2, 1, 8, [1, 3], [40, 9], 16),
    ("bs8_gqa8", 16, 2, 64, [1, 1], [200, 95], 8),
    ("bs32", 4, 4, 128, [1, 2], [300, 31], 32),
    ("bs1", 2, 2, 64, [1], [37], 1),
    ("group3_prefill", 6, 2, 64, [20, 1], [20, 60], 16),
    ("empty_query_seq", 4, 2, 64, [0, 1, 0, 3], [10, 20, 30, 40], 16),
]


@pytest.mark.parametrize("path", ["auto", "valu", "mfma"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pth_attention_parity(case, mode, path, monkeypatch):
    """Every case on the planner's choice and on each path forced (the matrix
    core path takes head sizes 64 and 128 with pages a multiple of 16;
    elsewhere the forced run falls back to the vector path)."""
    if path != "auto":
        monkeypatch.setenv("KV4_FORCE_PATH", path)
    name, nq, nkv, hs, ql, sl, bs = case
    _run(W.custom(name, nq, nkv, hs, ql, sl, block_size=bs), mode)


SCHED = {
    "streamk": {},
    "streamk_grid3": {"KV4_SK_GRID": "3"},
    "splits64": {"KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "64"},
    "split100": {"KV4_SPLIT_TOKENS": "100"},
    "streamk_nt_on": {"KV4_NT": "1"},
    "streamk_nt_off": {"KV4_NT": "0"},
}


@pytest.mark.parametrize("sched", list(SCHED))
@pytest.mark.parametrize("mode", MODES)
def test_pth_attention_schedules(mode, sched, monkeypatch):
    """Decode and mixed batches under each work schedule (stream-K pieces and
    split-KV partials, both merged by log-sum-exp)."""
    for k, v in SCHED[sched].items():
        monkeypatch.setenv(k, v)
    _run(W.custom("sched_decode", 32, 8, 128, [1] * 5, [1000, 17, 300, 2049, 64], block_size=16), mode)
    _run(W.custom("sched_decode64", 16, 4, 64, [1] * 4, [513, 1, 64, 700], block_size=32), mode)
    _run(W.custom("sched_mixed", 8, 2, 128, [1, 1, 7, 1], [1500, 63, 700, 1], block_size=16), mode)
    _run(W.custom("sched_mixed96", 8, 2, 96, [1, 1, 7, 1], [1500, 63, 700, 1], block_size=16), mode)
    _run(W.custom("sched_decode192", 8, 4, 192, [1] * 3, [700, 33, 1200], block_size=16), mode)
    _run(W.custom("sched_mha96", 8, 8, 96, [1] * 3, [900, 5, 260], block_size=32), mode)


@pytest.mark.parametrize("mode", MODES)
def test_pth_attention_custom_softmax_scale_and_outliers(mode):
    w = W.custom("outliers", 8, 2, 128, [1, 2], [700, 40], block_size=16, outlier_frac=0.05)
    _run(w, mode, softmax_scale=0.3)


@pytest.mark.parametrize("mode", MODES)
def test_pth_attention_vs_unquantized(mode):
    """The quantization error of the mode itself, against fp64 attention on
    the bf16 inputs."""
    w = W.custom("unquant", 8, 2, 128, [1, 1, 4], [2000, 300, 64], block_size=16)
    lay, key, value, query, got, _, sc = _run(w, mode)
    ref = O.attention_dense(query, key, value, lay.query_start_loc, lay.seq_lens, sc, lay.kv_start)
    nbad, mx = allclose_report(got, ref, **G4)
    c = corr(got, ref)
    say(f"    G4 {mode}: max abs err {mx:.3e}, violations {nbad}, corr {c:.6f}")
    assert c > 0.99
    if mode == "int8":
        assert nbad == 0, f"G4: {nbad} elements outside 5e-2 (max err {mx})"



@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("gain", [2.0 ** -30, 2.0 ** -8, 2.0 ** 6, 2.0 ** 40])
@pytest.mark.parametrize("mode", MODES)
def test_pth_attention_query_range(mode, gain, path, monkeypatch):
    """Queries far from unit size: flat and one-hot softmax rows, and q' rows
    whose power-of-two normalization (matrix-core path) moves them by up to
    2^40."""
    monkeypatch.setenv("KV4_FORCE_PATH", path)
    w = W.custom("qrange", 8, 2, 128, [1, 3, 1], [600, 80, 17], block_size=16)
    _run(w, mode, q_gain=gain)
