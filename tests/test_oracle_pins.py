"""Pins of the CPU oracle against facts fixed outside it: values printed on the
pages, hand-worked examples, closed forms, invariants and library routines.

A plausible mistake anywhere in the oracle (a dropped sign, a transposed H,
a divisor of head_size instead of b, a reversed butterfly order, the wrong
nibble order, a truncating instead of ties-to-even rounding) fails at least one
test here; test_planted_mistakes_are_caught checks that claim directly.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.special
import torch

from oracle import kv4_oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- D

def test_splitmix64_published_vectors():
    g = _gold("splitmix64_vectors.json")["outputs"]
    for seed, outs in g.items():
        want = [int(x, 0) for x in outs]
        assert O.splitmix64(int(seed), len(want)) == want


def test_signs_pm1_and_involution():
    for hs in (8, 96, 128, 192, 256):
        d = O.rht_signs(42, hs)
        assert set(np.unique(d)) <= {-1.0, 1.0}
        np.testing.assert_array_equal(d * d, np.ones(hs))          # D.D = I
    z = O.splitmix64(42, 4)
    np.testing.assert_array_equal(O.rht_signs(42, 4), [(-1.0 if v >> 63 else 1.0) for v in z])
    # both signs occur, roughly balanced
    d = O.rht_signs(7, 4096)
    assert abs(d.mean()) < 0.1


# ------------------------------------------------------------------------ H, b

def test_b_rule_closed_form():
    assert [O.largest_pow2_divisor(h) for h in (128, 96, 64, 192, 80, 120, 256)] == \
        [128, 32, 64, 64, 16, 8, 256]
    for hs in range(1, 513):
        b = O.largest_pow2_divisor(hs)
        assert hs % b == 0 and (hs // b) % 2 == 1
        assert (b == hs) == (hs & (hs - 1) == 0)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_equals_scipy_sylvester(b):
    np.testing.assert_array_equal(O.hadamard(b), scipy.linalg.hadamard(b).astype(np.float64))


@pytest.mark.parametrize("hs", [8, 64, 80, 96, 128, 192, 256])
def test_block_diag_orthogonal_up_to_b(hs):
    H = O.block_diag_hadamard(hs)
    b = O.largest_pow2_divisor(hs)
    np.testing.assert_array_equal(H @ H.T, b * np.eye(hs))
    np.testing.assert_array_equal(H, H.T)
    # no mixing across blocks
    mask = np.kron(np.eye(hs // b), np.ones((b, b))).astype(bool)
    assert not H[~mask].any()


def test_hadamard_worked_examples():
    g = _gold("hadamard_worked.json")
    x = np.array(g["sylvester_4"]["x"], float)
    np.testing.assert_array_equal(O.hadamard(4) @ x, g["sylvester_4"]["Hx"])
    x = np.array(g["block_diag_12_b4"]["x"], float)
    np.testing.assert_array_equal(O.block_diag_hadamard(12) @ x, g["block_diag_12_b4"]["Hx"])
    np.testing.assert_array_equal(O.fwht_spec_f32(x.astype(np.float32), 4), g["block_diag_12_b4"]["Hx"])


def test_butterfly_stage_order_worked_example():
    g = _gold("hadamard_worked.json")["stage_order_fp32"]
    x = np.array(g["x"], dtype=np.float32)
    y = O.fwht_spec_f32(x, 4)
    assert y[0] == np.float32(g["y0_ascending"])
    assert (O.hadamard(4) @ x.astype(np.float64))[0] == g["y0_exact"]


@pytest.mark.parametrize("hs", [16, 96, 128, 192])
def test_rotation_roundtrip_identity(hs):
    rng = np.random.default_rng(hs)
    x = rng.standard_normal((5, hs))
    d = O.rht_signs(3, hs)
    np.testing.assert_allclose(O.unrotate_math(O.rotate_math(x, d), d), x, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hs", [64, 96, 128, 192])
def test_score_preservation(hs):
    """q'.K_s / b = q.k for the unquantized rotation."""
    rng = np.random.default_rng(hs + 1)
    q = rng.standard_normal((7, hs))
    k = rng.standard_normal((9, hs))
    d = O.rht_signs(11, hs)
    b = O.largest_pow2_divisor(hs)
    lhs = O.rotate_math(q, d) @ O.rotate_math(k, d).T / b
    np.testing.assert_allclose(lhs, q @ k.T, rtol=0, atol=1e-10)


@pytest.mark.parametrize("hs", [32, 96, 128, 192, 256])
def test_fwht_spec_exact_on_small_integers(hs):
    """Integer inputs small enough that every float32 partial sum is exact:
    the butterfly must equal the dense matrix product exactly."""
    rng = np.random.default_rng(hs)
    x = rng.integers(-1000, 1000, size=(20, hs)).astype(np.float32)
    b = O.largest_pow2_divisor(hs)
    np.testing.assert_array_equal(O.fwht_spec_f32(x, b), x.astype(np.float64) @ O.block_diag_hadamard(hs).T)


@pytest.mark.parametrize("hs", [96, 128, 192])
def test_fwht_spec_error_bound(hs):
    """Each output is built by log2(b) levels of float32 add/sub: error is at
    most log2(b) * 2^-24 * sum|x| of its block (first order)."""
    rng = np.random.default_rng(hs + 5)
    x = rng.standard_normal((200, hs)).astype(np.float32) * np.float32(3)
    b = O.largest_pow2_divisor(hs)
    y = O.fwht_spec_f32(x, b).astype(np.float64)
    ref = x.astype(np.float64) @ O.block_diag_hadamard(hs).T
    blk_abs = np.abs(x.astype(np.float64)).reshape(200, hs // b, b).sum(-1)
    bound = math.log2(b) * 2.0 ** -24 * np.repeat(blk_abs, b, axis=1) * 1.0001
    assert np.all(np.abs(y - ref) <= bound)


# ------------------------------------------------------------------------ bf16

def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    # exact ties: bf16 value + half an ulp, both parities
    base = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16).to(torch.float32).numpy()
    u = base.view(np.uint32) | np.uint32(0x8000)
    ties = u.view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.bf16_round(x).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("hs", [128, 96, 192])
def test_rotation_bf16_error_matches_pages_order(hs):
    """The stored rotation vs an fp64 block-diagonal reference: per element
    within bf16's half-ulp (2^-8 relative) plus the float32 butterfly error,
    and the aggregate relative error of the same order as the pages' figures
    (3.56e-3 / 3.99e-3 / 3.52e-3 for head_size 128 / 96 / 192)."""
    page = _gold("pages_values.json")["rht_relative_error_vs_fp64_blockdiag"]["values"][str(hs)]
    x = W.normal_bf16((4096, hs), seed=hs).to(torch.float32).numpy()
    d = O.rht_signs(42, hs)
    ys = O.rotate_spec(x, d).astype(np.float64)
    y64 = O.rotate_math(x, d)
    b = O.largest_pow2_divisor(hs)
    slack = math.log2(b) * 2.0 ** -24 * np.abs(x).sum(-1, keepdims=True) * 2
    assert np.all(np.abs(ys - y64) <= 2.0 ** -8 * np.abs(y64) + slack)
    maxrel = np.max(np.abs(ys - y64)) / np.max(np.abs(y64))
    assert 0.25 * page <= maxrel <= 2.0 * page, (maxrel, page)


def test_unrotated_entries_std_matches_pages():
    """D.H.k/b of an unrotated k ~ N(0,1) has std 1/sqrt(b) (pages: about
    1/sqrt(128) at head_size 128)."""
    g = _gold("pages_values.json")["unrotated_entry_std"]
    hs = g["head_size"]
    rng = np.random.default_rng(1)
    k = rng.standard_normal((4000, hs))
    s = O.unrotate_math(k, O.rht_signs(42, hs)).std()
    assert abs(s - g["value"]) < 0.02 * g["value"]


# -------------------------------------------------------------------- quantizer

def test_quantizer_worked_examples():
    g = _gold("int4_worked.json")
    for c in g["cases"]:
        codes, scale = O.quantize_int4(np.array(c["y"], np.float32))
        assert scale == np.float32(c["scale"])
        np.testing.assert_array_equal(codes, c["codes"])
        np.testing.assert_array_equal(O.pack_int4(codes), [int(b, 0) for b in c["bytes"]])
    for p in g["pack_pairs"]:
        assert O.pack_int4(np.array(p["codes"]))[0] == int(p["byte"], 0)
        np.testing.assert_array_equal(O.unpack_int4(np.array([int(p["byte"], 0)], np.uint8)), p["codes"])


def test_pack_unpack_all_bytes():
    allb = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(O.pack_int4(O.unpack_int4(allb)), allb)


def _rne_fraction(f: Fraction) -> int:
    fl = math.floor(f)
    r = f - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("hs", [2, 4, 6, 8, 12])
def test_quantizer_brute_force_tiny(hs):
    """Exact rational arithmetic: scale is the float32 rounding of amax/7, and
    every code is the integer in [-8, 7] nearest to y/scale (ties to even),
    computed by trying all 16 codes."""
    rng = np.random.default_rng(hs)
    for _ in range(300):
        y = (rng.standard_normal(hs) * 4).astype(np.float32)
        codes, scale = O.quantize_int4(y)
        amax = max(abs(Fraction(float(v))) for v in y)
        assert scale == np.float32(float(amax / 7))
        for v, c in zip(y, codes):
            q = Fraction(float(v)) / Fraction(float(scale))
            best = min(range(-8, 8), key=lambda k: (abs(q - k), k % 2))
            assert _rne_fraction(q) == best
            assert int(c) == best
        assert np.all(np.abs(codes) <= 7)


def test_quantizer_zero_and_bounds():
    codes, scale = O.quantize_int4(np.zeros((3, 16), np.float32))
    assert np.all(scale == 0) and np.all(codes == 0)
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((1000, 128)) * 10).astype(np.float32)
    codes, scale = O.quantize_int4(y)
    assert codes.min() >= -7 and codes.max() <= 7
    err = np.abs(codes * scale[:, None].astype(np.float64) - y)
    assert np.all(err <= scale[:, None] * (0.5 + 1e-6))


def test_roundtrip_rms_closed_form():
    """Round trip k -> cache -> D.H(.)/b: the per-element error rms is
    E[scale]/sqrt(12)/sqrt(b) with scale = amax/7 and amax the max of hs
    |N(0, b)| draws, i.e. E[max_i |g_i|] / (7 sqrt(12)) for g ~ N(0, 1)."""
    hs = 128
    n = hs
    emax = scipy.integrate.quad(lambda x: 1.0 - scipy.special.erf(x / math.sqrt(2)) ** n, 0, 20)[0]
    want = emax / (7 * math.sqrt(12))
    x = W.normal_bf16((4000, 1, hs), seed=9).to(torch.float32).numpy()
    slots = np.arange(4000)
    kc, ks = O.new_cache(4000 // 16, 16, 1, hs)
    O.rht_write(x, kc, ks, slots, 42)
    back = O.dequant(kc, ks, slots, 42, inverse_rotate=True)
    rms = np.sqrt(np.mean((back - x) ** 2))
    assert abs(rms - want) < 0.05 * want, (rms, want)
    # the pages' elementwise tolerance 0.5 + 0.5|x| holds except for a ~1e-5 tail
    tol = _gold("pages_values.json")["dequant_tolerance"]
    bad = np.abs(back - x) > tol["atol"] + tol["rtol"] * np.abs(x)
    assert bad.mean() < 1e-4


def test_kv_footprint_roughly_4x():
    g = _gold("pages_values.json")["kv_footprint"]
    for hs in (96, 128):
        ratio = (4 * hs) / (hs + 8)
        assert abs(ratio - g["ratio_approx"]) < 0.35


def test_write_dequant_layout_and_skip():
    """Slot -> (slot // bs, slot % bs), negative slots untouched, dequant of
    the stored codes is code * scale in one float32 product."""
    hs, nkv, bs = 96, 3, 16
    x = W.normal_bf16((40, nkv, hs), seed=2).to(torch.float32).numpy()
    slots = np.arange(40) * 3 % 128
    slots[5] = -1
    kc, ks = O.new_cache(8, bs, nkv, hs)
    O.rht_write(x, kc, ks, slots, 42)
    blk, off = slots[5 + 0] // bs, slots[5] % bs
    used = set(int(s) for s in slots if s >= 0)
    for s in range(128):
        if s not in used:
            assert not kc[s // bs, s % bs].any() and not ks[s // bs, s % bs].any()
    t = 7
    y = O.rotate_spec(x[t], O.rht_signs(42, hs))
    codes, scale = O.quantize_int4(y)
    np.testing.assert_array_equal(kc[slots[t] // bs, slots[t] % bs], O.pack_int4(codes))
    deq = O.dequant(kc, ks, slots[t:t + 1], 42, inverse_rotate=False)[0]
    np.testing.assert_array_equal(deq, (codes.astype(np.float32) * scale[:, None]).astype(np.float32))


# -------------------------------------------------------------------- attention

def _sdpa_reference(q, k, v, query_lens, seq_lens, kv_start, scale):
    """torch scaled_dot_product_attention (fp64, CPU) with an explicit causal
    offset mask, per sequence and kv-head group."""
    out = np.zeros(q.shape)
    nq, nkv = q.shape[1], k.shape[1]
    grp = nq // nkv
    q0 = 0
    for s, (ql, L) in enumerate(zip(query_lens, seq_lens)):
        k0 = kv_start[s]
        qs = torch.from_numpy(q[q0:q0 + ql]).permute(1, 0, 2)            # [nq, ql, hs]
        ks = torch.from_numpy(np.repeat(k[k0:k0 + L], grp, axis=1)).permute(1, 0, 2)
        vs = torch.from_numpy(np.repeat(v[k0:k0 + L], grp, axis=1)).permute(1, 0, 2)
        pos = L - ql + torch.arange(ql)
        mask = torch.arange(L)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=scale)
        out[q0:q0 + ql] = o.permute(1, 0, 2).numpy()
        q0 += ql
    return out


def test_attention_dense_matches_sdpa():
    rng = np.random.default_rng(3)
    qlens, slens = [1, 5, 3, 1], [17, 40, 3, 1]
    hs, nq, nkv = 64, 6, 2
    q = rng.standard_normal((sum(qlens), nq, hs))
    k = rng.standard_normal((sum(slens), nkv, hs))
    v = rng.standard_normal((sum(slens), nkv, hs))
    kvs = np.concatenate([[0], np.cumsum(slens)])
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    got = O.attention_dense(q, k, v, qsl, slens, hs ** -0.5, kvs)
    want = _sdpa_reference(q, k, v, qlens, slens, kvs, hs ** -0.5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def _small_case(hs=96, nq=8, nkv=2, qlens=(1, 4, 1), slens=(37, 50, 16), seed=0):
    w = W.custom("t", nq, nkv, hs, qlens, slens, seed=seed)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    key, value, query = (W.bf16_as_f32_numpy(x) for x in (t.key, t.value, t.query))
    slots = W.all_slots(lay, w)
    caches = O.write_kv(key, value, slots, lay.num_blocks, w.block_size, w.sign_seed)
    return w, lay, key, value, query, slots, caches


@pytest.mark.parametrize("hs", [96, 128])
def test_rotated_form_equals_original_domain(hs):
    """Rotated attention on the int4 cache (q' = H.D.q, softmax_scale / b,
    output D.H(.)/b) equals plain attention on the dequantized, inverse-rotated
    K/V -- the compensation identities of the read path."""
    w, lay, key, value, query, slots, (kc, vc, ks, vs) = _small_case(hs=hs)
    sc = hs ** -0.5
    got = O.paged_attention(query, kc, vc, ks, vs, lay.block_table, lay.seq_lens,
                            lay.query_start_loc, sc, w.sign_seed)
    bs = w.block_size
    d = O.rht_signs(w.sign_seed, hs)

    def exact_dequant(c, sc):   # code * scale in fp64, then D.H(.)/b
        y = O.unpack_int4(c[slots // bs, slots % bs]).astype(np.float64)
        return O.unrotate_math(y * sc[slots // bs, slots % bs].astype(np.float64)[..., None], d)

    kh, vh = exact_dequant(kc, ks), exact_dequant(vc, vs)
    want = O.attention_dense(query, kh, vh, lay.query_start_loc, w.seq_lens, sc, lay.kv_start)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def test_output_std_matches_pages():
    """Reference output std with 4 heads, head_size 128, N(0,1) q/k/v: about
    0.15 at kv_len 128 and 0.25-0.3 at kv_len 64 and 32."""
    g = _gold("pages_values.json")["reference_output_std"]
    res = {}
    for L in (32, 64, 128):
        vals = []
        for seed in range(40):
            rng = np.random.default_rng(seed)
            q = rng.standard_normal((1, 4, 128))
            k = rng.standard_normal((L, 4, 128))
            v = rng.standard_normal((L, 4, 128))
            o = O.attention_dense(q, k, v, [0, 1], [L], 128 ** -0.5, [0, L])
            vals.append(o.std())
        res[L] = float(np.mean(vals))
    assert abs(res[128] - g["kv_len_128"]) < 0.02
    lo, hi = g["kv_len_64_32_range"]
    assert lo - 0.06 <= res[64] <= hi and lo - 0.06 <= res[32] <= hi + 0.03
    # closed form sqrt(e / L) for softmax of N(0,1) logits
    for L in (32, 64, 128):
        assert abs(res[L] - math.sqrt(math.e / L)) < 0.08 * math.sqrt(math.e / L) + 0.005


def test_negative_control_unrotated_cache():
    """Filling the int4 cache with unrotated K/V (quantized without H.D) and
    reading it with the rotated read path gives an output near 0 that is
    uncorrelated with the reference (the pages' failure before the fix)."""
    hs, L = 128, 128
    rng = np.random.default_rng(0)
    q = W.normal_bf16((1, 4, hs), seed=100).to(torch.float32).numpy()
    k = W.normal_bf16((L, 4, hs), seed=101).to(torch.float32).numpy()
    v = W.normal_bf16((L, 4, hs), seed=102).to(torch.float32).numpy()
    kc, ks = O.new_cache(L // 16, 16, 4, hs)
    vc, vs = O.new_cache(L // 16, 16, 4, hs)
    for x, c, sc in ((k, kc, ks), (v, vc, vs)):
        codes, scale = O.quantize_int4(x)              # no rotation
        c[:] = O.pack_int4(codes).reshape(c.shape)
        sc[:] = scale.reshape(sc.shape)
    bt = np.arange(L // 16, dtype=np.int32)[None]
    out = O.paged_attention(q, kc, vc, ks, vs, bt, [L], [0, 1], hs ** -0.5, 42)
    ref = O.attention_dense(q, k, v, [0, 1], [L], hs ** -0.5, [0, L])
    corr = np.corrcoef(out.ravel(), ref.ravel())[0, 1]
    assert abs(corr) < 0.2
    assert out.std() < 0.2 * ref.std()
    # with the rotation the same data tracks the unquantized reference (up to
    # the int4 error itself, which is large at kv_len 128)
    slots = np.arange(L)
    kc2, vc2, ks2, vs2 = O.write_kv(k, v, slots, L // 16, 16, 42)
    out2 = O.paged_attention(q, kc2, vc2, ks2, vs2, bt, [L], [0, 1], hs ** -0.5, 42)
    assert np.corrcoef(out2.ravel(), ref.ravel())[0, 1] > 0.95


def test_int4_attention_within_pages_tolerance_where_achievable():
    """At head_size 64 and kv_len 2560 the int4 error of the method itself is
    well inside the pages' atol = rtol = 5e-2 against unquantized attention."""
    tol = _gold("pages_values.json")["attention_tolerance"]
    for seed in (0, 1):
        w, lay, key, value, query, slots, (kc, vc, ks, vs) = _small_case(
            hs=64, nq=4, nkv=1, qlens=(1, 1), slens=(2560, 2000), seed=seed)
        sc = 64 ** -0.5
        got = O.paged_attention(query, kc, vc, ks, vs, lay.block_table, lay.seq_lens,
                                lay.query_start_loc, sc, w.sign_seed)
        ref = O.attention_dense(query, key, value, lay.query_start_loc, w.seq_lens, sc, lay.kv_start)
        np.testing.assert_allclose(got, ref, atol=tol["atol"], rtol=tol["rtol"])


# ---------------------------------------------------------- planted mistakes

def _pins_pass() -> bool:
    """Re-run a subset of the pins; False if any fails."""
    checks = [
        test_hadamard_worked_examples, test_butterfly_stage_order_worked_example,
        lambda: test_rotation_roundtrip_identity(96), lambda: test_score_preservation(96),
        test_quantizer_worked_examples, lambda: test_quantizer_brute_force_tiny(8),
        lambda: test_rotated_form_equals_original_domain(96),
        test_negative_control_unrotated_cache, test_splitmix64_published_vectors,
        lambda: test_hadamard_equals_scipy_sylvester(8),
    ]
    for c in checks:
        try:
            c()
        except Exception:   # an assertion, or the planted code failing outright
            return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass()
    real_fwht = O.fwht_spec_f32
    real_b = O.largest_pow2_divisor
    real_pack = O.pack_int4
    real_rotate = O.rotate_math
    real_hadamard = O.hadamard
    real_sm = O.splitmix64

    def descending(x, b):       # butterfly strides in the wrong order
        y = np.array(x, dtype=np.float32, copy=True)
        d = y.shape[-1]
        v = y.reshape(y.shape[:-1] + (d // b, b))
        h = b // 2
        while h >= 1:
            w = v.reshape(v.shape[:-1] + (b // (2 * h), 2, h))
            lo, hi = w[..., 0, :].copy(), w[..., 1, :].copy()
            w[..., 0, :], w[..., 1, :] = lo + hi, lo - hi
            h //= 2
        return v.reshape(y.shape)

    def high_first(codes):      # nibble order swapped
        c = np.asarray(codes, dtype=np.int16) & 0xF
        return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)

    def dh_order(x, signs):     # D applied after H
        H = O.block_diag_hadamard(x.shape[-1])
        return (np.asarray(x, dtype=np.float64) @ H.T) * signs

    def transposed_bitrev(b):   # a Hadamard in another row order
        H = real_hadamard(b)
        return H[::-1].copy()

    def off_by_one_sm(seed, n):
        return real_sm(seed + 1, n)

    mistakes = [
        ("fwht_spec_f32", descending),
        ("largest_pow2_divisor", lambda n: n),
        ("pack_int4", high_first),
        ("rotate_math", dh_order),
        ("hadamard", transposed_bitrev),
        ("splitmix64", off_by_one_sm),
    ]
    for name, fake in mistakes:
        with monkeypatch.context() as m:
            m.setattr(O, name, fake)
            assert not _pins_pass(), f"planted mistake in {name} not caught"
    assert _pins_pass()


# ---------------------------------------------------------------------------
# Sliding window (a reading of the pages' "added window" commit: the query at
# position p sees keys j with p - W < j <= p)
# ---------------------------------------------------------------------------

def _window_case(seed=0):
    rng = np.random.default_rng(seed)
    nq, nkv, hs = 4, 2, 16
    slens, qlens = [37, 9, 20], [1, 3, 5]
    q = rng.standard_normal((sum(qlens), nq, hs))
    k = rng.standard_normal((sum(slens), nkv, hs))
    v = rng.standard_normal((sum(slens), nkv, hs))
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    kv_start = np.concatenate([[0], np.cumsum(slens)])
    return q, k, v, qsl, np.array(slens), kv_start


def test_window_degenerate_cases_reduce_to_causal_and_to_self():
    q, k, v, qsl, sl, ks = _window_case()
    causal = O.attention_dense(q, k, v, qsl, sl, 0.25, ks)
    # a window at least as long as every sequence changes nothing
    assert np.array_equal(O.attention_dense(q, k, v, qsl, sl, 0.25, ks, window=int(sl.max())), causal)
    assert np.array_equal(O.attention_dense(q, k, v, qsl, sl, 0.25, ks, window=0), causal)
    # window 1: every query sees only its own key, so the output is its own value row
    w1 = O.attention_dense(q, k, v, qsl, sl, 0.25, ks, window=1)
    group = q.shape[1] // k.shape[1]
    for s in range(len(sl)):
        L, q0, q1 = int(sl[s]), int(qsl[s]), int(qsl[s + 1])
        for i in range(q1 - q0):
            pos = L - (q1 - q0) + i
            for h in range(q.shape[1]):
                assert np.allclose(w1[q0 + i, h], v[ks[s] + pos, h // group], atol=1e-12)


@pytest.mark.parametrize("W", [2, 5, 8, 19])
def test_window_equals_causal_attention_on_the_truncated_history(W):
    """Each row's windowed result equals plain causal attention of that row
    over only its last W keys (slicing instead of masking)."""
    q, k, v, qsl, sl, ks = _window_case(seed=W)
    got = O.attention_dense(q, k, v, qsl, sl, 0.25, ks, window=W)
    for s in range(len(sl)):
        L, q0, q1 = int(sl[s]), int(qsl[s]), int(qsl[s + 1])
        for i in range(q1 - q0):
            pos = L - (q1 - q0) + i
            lo = max(0, pos - W + 1)
            n = pos + 1 - lo                       # keys lo .. pos, the row is the last query
            ref = O.attention_dense(q[q0 + i:q0 + i + 1], k[ks[s] + lo:ks[s] + pos + 1],
                                    v[ks[s] + lo:ks[s] + pos + 1], np.array([0, 1]), np.array([n]), 0.25,
                                    np.array([0, n]))
            assert np.allclose(got[q0 + i], ref[0], atol=1e-12)


def test_window_paged_forms_agree_with_dense():
    """The paged oracles (int4 rotated domain and int8) pass the window to the
    same mask: their windowed results match dense windowed attention on the
    dequantized values."""
    rng = np.random.default_rng(4)
    nq, nkv, hs, bs = 4, 2, 32, 4
    slens, qlens = [23, 10], [1, 4]
    T = sum(slens)
    key = rng.standard_normal((T, nkv, hs)).astype(np.float32)
    value = rng.standard_normal((T, nkv, hs)).astype(np.float32)
    q = rng.standard_normal((sum(qlens), nq, hs))
    nb = 16
    bt = np.full((2, 8), -1, dtype=np.int32)
    perm = rng.permutation(nb)
    slots, kv_start, used = [], [0], 0
    for s, L in enumerate(slens):
        n = -(-L // bs)
        bt[s, :n] = perm[used:used + n]
        used += n
        slots += [int(bt[s, p // bs]) * bs + p % bs for p in range(L)]
        kv_start.append(kv_start[-1] + L)
    slots = np.array(slots, dtype=np.int64)
    qsl = np.array([0, 1, 5])
    sl = np.array(slens)
    kc, vc, ks, vs = O.pth_write_kv(key, value, slots, nb, bs, "int8")
    kd = O.pth_dequant(kc, ks, slots, "int8").astype(np.float64)
    vd = O.pth_dequant(vc, vs, slots, "int8").astype(np.float64)
    for W in (1, 3, 7):
        got = O.pth_paged_attention(q, kc, vc, ks, vs, bt, sl, qsl, 0.2, "int8", window=W)
        ref = O.attention_dense(q, kd, vd, qsl, sl, 0.2, np.array(kv_start), window=W)
        assert np.allclose(got, ref, atol=1e-6)
        kc4, vc4, ks4, vs4 = O.write_kv(key, value, slots, nb, bs, 42)
        got4 = O.paged_attention(q, kc4, vc4, ks4, vs4, bt, sl, qsl, 0.2, 42, window=W)
        kh = O.dequant(kc4, ks4, slots, 42, inverse_rotate=True).astype(np.float64)
        vh = O.dequant(vc4, vs4, slots, 42, inverse_rotate=True).astype(np.float64)
        ref4 = O.attention_dense(q, kh, vh, qsl, sl, 0.2, np.array(kv_start), window=W)
        assert np.allclose(got4, ref4, atol=1e-4)


def test_empty_causal_window_rows_are_zero():
    """A sequence shorter than its query block leaves its first rows with no
    visible key (position < 0): the oracle returns exactly 0 there, with no
    NaN and no floating-point warning, and every other row equals causal
    attention computed over the rows that do see keys. A sequence of length
    0 gives all-zero rows. Same reading in the dense, int4 and int8 forms."""
    import warnings
    rng = np.random.default_rng(11)
    nq, nkv, hs = 4, 2, 32
    qlens, slens = [5, 2, 1], [3, 0, 6]
    q = rng.standard_normal((sum(qlens), nq, hs))
    k = rng.standard_normal((sum(slens), nkv, hs))
    v = rng.standard_normal((sum(slens), nkv, hs))
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    kvs = np.concatenate([[0], np.cumsum(slens)])
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        got = O.attention_dense(q, k, v, qsl, slens, 0.3, kvs)
        gotw = O.attention_dense(q, k, v, qsl, slens, 0.3, kvs, window=2)
    assert np.isfinite(got).all() and np.isfinite(gotw).all()
    # sequence 0: rows at positions -2, -1 see nothing; rows 2..4 see keys 0..i-2
    assert not got[0:2].any() and not gotw[0:2].any()
    # sequence 1 (length 0): both rows are zero
    assert not got[5:7].any()
    # the rows with keys equal attention over a query block of the same positions
    tail = O.attention_dense(q[2:5], k[0:3], v[0:3], np.array([0, 3]), [3], 0.3, np.array([0, 3]))
    np.testing.assert_allclose(got[2:5], tail, rtol=0, atol=1e-14)
    want = _sdpa_reference(q[2:5], k[0:3], v[0:3], [3], [3], np.array([0, 3]), 0.3)
    np.testing.assert_allclose(got[2:5], want, rtol=1e-12, atol=1e-12)

    # paged forms over caches written by the oracle
    bs, nb = 4, 6
    bt = np.zeros((3, 2), dtype=np.int32)
    bt[0, 0] = 0
    bt[2, :] = [1, 2]
    slots = np.array([0, 1, 2] + [4, 5, 6, 7, 8, 9], dtype=np.int64)
    key32, val32 = k.astype(np.float32), v.astype(np.float32)
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        kc, vc, ks, vs = O.write_kv(key32, val32, slots, nb, bs, 42)
        p4 = O.paged_attention(q, kc, vc, ks, vs, bt, np.array(slens), qsl, 0.3, 42)
        kc8, vc8, ks8, vs8 = O.pth_write_kv(key32, val32, slots, nb, bs, "int8")
        p8 = O.pth_paged_attention(q, kc8, vc8, ks8, vs8, bt, np.array(slens), qsl, 0.3, "int8")
    for p in (p4, p8):
        assert np.isfinite(p).all()
        assert not p[0:2].any() and not p[5:7].any()
        assert np.abs(p[2:5]).max() > 0.05 and np.abs(p[7]).max() > 0.05
