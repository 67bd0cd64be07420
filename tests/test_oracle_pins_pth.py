"""Pins of the oracle's per-token-head INT8 / FP8 control modes (no rotation).

Each check compares the oracle with something other than itself: torch's own
float8_e4m3fn conversion (an independent implementation of the OCP FP8 E4M3
format), hand-derived worked examples from the format definition, closed forms,
brute force over exact rationals, and the oracle's separately pinned dense
attention on the dequantized values. A planted mistake in each function must be
caught.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kv4_oracle as O


def _torch_fp8_bytes(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3fn_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    # format facts: 0x7E = 448 is the largest finite value, 0x01 = 2^-9 the smallest subnormal
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_fp8_encode_matches_torch_on_values_midpoints_and_random():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.fp8_e4m3fn_decode(codes)
    fin = ~np.isnan(vals)
    # every representable value encodes to itself
    assert np.array_equal(O.fp8_e4m3fn_encode(vals[fin].astype(np.float32)), codes[fin])
    # ties (midpoints of neighbours) round to the even mantissa, as torch does
    pos = np.sort(vals[fin & (codes < 0x80)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(O.fp8_e4m3fn_encode(mids), _torch_fp8_bytes(mids))
    assert np.array_equal(O.fp8_e4m3fn_encode(-mids), _torch_fp8_bytes(-mids))
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-14, 6, 100000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(O.fp8_e4m3fn_encode(x), _torch_fp8_bytes(x))


def test_fp8_encode_worked_examples():
    # hand-derived from the format definition (sign, 4-bit exponent bias 7, 3-bit mantissa)
    cases = [(448.0, 0x7E), (-448.0, 0xFE), (449.0, 0x7E), (1e6, 0x7E), (1.0, 0x38), (1.5, 0x3C),
             (0.0, 0x00), (-0.0, 0x80), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (224.0, 0x76), (112.0, 0x6E), (240.0, 0x77), (232.0, 0x76)]
    for v, c in cases:
        assert int(O.fp8_e4m3fn_encode(np.array([v], np.float32))[0]) == c, v


def test_quantize_pth_worked_examples():
    c, s = O.quantize_pth(np.array([[127.0, -127.0, 63.5, 0.49]], np.float32), "int8")
    assert s[0] == np.float32(1.0)
    assert list(c[0].view(np.int8)) == [127, -127, 64, 0]        # 63.5 -> 64 (half to even)
    c, s = O.quantize_pth(np.array([[1.0, -2.0, 0.5]], np.float32), "fp8")
    assert s[0] == np.float32(2.0) / np.float32(448.0)
    assert [int(v) for v in c[0]] == [0x76, 0xFE, 0x6E]         # 224, -448, 112
    for mode in ("int8", "fp8"):
        c, s = O.quantize_pth(np.zeros((2, 16), np.float32), mode)
        assert (s == 0).all() and (c == 0).all()


def test_int8_quantizer_brute_force():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 24)) * 3).astype(np.float32)
    codes, scale = O.quantize_pth(x, "int8")
    for r in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[r])
        s = np.float32(np.float32(amax) / np.float32(127.0))
        assert scale[r] == s
        for j in range(x.shape[1]):
            q = Fraction(float(np.float32(x[r, j] / s)))                 # the float32 quotient, exactly
            fl = q.numerator // q.denominator
            rem = q - fl
            rn = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            assert int(codes[r, j].view(np.int8)) == max(-128, min(127, rn))


def test_pth_roundtrip_error_bounds():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((512, 4, 128)).astype(np.float32)
    slots = np.arange(512)
    for mode, rel in (("int8", 0.5 / 127), ("fp8", 2.0 ** -4)):
        kc, ks = O.pth_new_cache(32, 16, 4, 128)
        O.pth_write(x, kc, ks, slots, mode)
        y = O.pth_dequant(kc, ks, slots, mode)
        amax = np.abs(x).max(axis=-1, keepdims=True)
        err = np.abs(y - x)
        if mode == "int8":
            # absolute error at most half a step (plus float32 rounding)
            assert (err <= amax * rel * (1 + 1e-5) + 1e-7).all()
        else:
            # relative error of a normal e4m3 value: at most 2^-4 of |x|; below the
            # normal range at most half the subnormal step
            scale = amax / 448.0
            assert (err <= np.maximum(np.abs(x) * rel, scale * 2.0 ** -10) * (1 + 1e-5) + 1e-7).all()


def test_pth_write_layout_and_skip():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 2, 16)).astype(np.float32)
    kc, ks = O.pth_new_cache(2, 4, 2, 16)
    slots = np.array([7, -1, 0, 8, 3])                 # 8 = nb * bs is outside, skipped
    O.pth_write(x, kc, ks, slots, "int8")
    c0, s0 = O.quantize_pth(x[0], "int8")
    assert np.array_equal(kc[1, 3], c0) and np.array_equal(ks[1, 3], s0)
    c2, s2 = O.quantize_pth(x[2], "int8")
    assert np.array_equal(kc[0, 0], c2)
    assert (kc[0, 1] == 0).all() and (ks[0, 2] == 0).all()


def _pth_case(mode, hs=64, nq=8, nkv=2, qlens=(1, 3, 1), slens=(33, 20, 1), seed=0):
    rng = np.random.default_rng(seed)
    T = sum(slens)
    key = rng.standard_normal((T, nkv, hs)).astype(np.float32)
    value = rng.standard_normal((T, nkv, hs)).astype(np.float32)
    query = rng.standard_normal((sum(qlens), nq, hs)).astype(np.float32)
    bs = 8
    nblk = [-(-L // bs) for L in slens]
    num_blocks = sum(nblk) + 1
    perm = rng.permutation(num_blocks)
    bt = np.zeros((len(slens), max(nblk)), np.int32)
    slots, kv_start, k = [], [], 0
    for s, L in enumerate(slens):
        bt[s, :nblk[s]] = perm[k:k + nblk[s]]
        k += nblk[s]
        kv_start.append(len(slots))
        slots += [int(bt[s, p // bs]) * bs + p % bs for p in range(L)]
    slots = np.array(slots)
    kc, vc, ks, vs = O.pth_write_kv(key, value, slots, num_blocks, bs, mode)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    return query, key, value, kc, vc, ks, vs, bt, np.array(slens), qsl, slots, np.array(kv_start)


@pytest.mark.parametrize("mode", ["int8", "fp8"])
def test_pth_attention_equals_dense_on_dequantized(mode):
    q, k, v, kc, vc, ks, vs, bt, sl, qsl, slots, kv_start = _pth_case(mode)
    got = O.pth_paged_attention(q, kc, vc, ks, vs, bt, sl, qsl, 0.125, mode)
    bs = kc.shape[1]
    # fp64 dequantized rows in slot order (code value * scale without a float32 rounding)
    kd = O.decode_pth(kc[slots // bs, slots % bs], mode) * ks[slots // bs, slots % bs].astype(np.float64)[..., None]
    vd = O.decode_pth(vc[slots // bs, slots % bs], mode) * vs[slots // bs, slots % bs].astype(np.float64)[..., None]
    ref = O.attention_dense(q, kd, vd, qsl, sl, 0.125, kv_start)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_pth_attention_closed_forms():
    q, k, v, kc, vc, ks, vs, bt, sl, qsl, slots, _ = _pth_case("int8", slens=(1, 20, 9), qlens=(1, 1, 1))
    # a single key: the output is that key's dequantized value row
    out = O.pth_paged_attention(q, kc, vc, ks, vs, bt, sl, qsl, 0.125, "int8")
    bs = vc.shape[1]
    vrow = O.decode_pth(vc[slots[0] // bs, slots[0] % bs], "int8") * vs[slots[0] // bs, slots[0] % bs][:, None]
    assert np.allclose(out[0], np.repeat(vrow, 4, axis=0), atol=1e-12)
    # a zero query: uniform weights, the output is the mean of the visible values
    q0 = np.zeros_like(q)
    out = O.pth_paged_attention(q0, kc, vc, ks, vs, bt, sl, qsl, 0.125, "int8")
    sl1 = slots[1:21]
    vseq = O.decode_pth(vc[sl1 // bs, sl1 % bs], "int8") * vs[sl1 // bs, sl1 % bs].astype(np.float64)[..., None]
    assert np.allclose(out[1], np.repeat(vseq.mean(axis=0), 4, axis=0), atol=1e-12)


def _pth_pins_pass() -> bool:
    checks = [test_fp8_decode_all_codes_match_torch, test_fp8_encode_matches_torch_on_values_midpoints_and_random,
              test_fp8_encode_worked_examples, test_quantize_pth_worked_examples, test_int8_quantizer_brute_force,
              test_pth_roundtrip_error_bounds, lambda: test_pth_attention_equals_dense_on_dequantized("fp8"),
              test_pth_attention_closed_forms, test_pth_write_layout_and_skip]
    for c in checks:
        try:
            c()
        except Exception:
            return False
    return True


def test_planted_mistakes_in_pth_oracle_are_caught(monkeypatch):
    assert _pth_pins_pass()
    real_enc, real_dec, real_q = O.fp8_e4m3fn_encode, O.fp8_e4m3fn_decode, O.quantize_pth

    def enc_truncating(x):                          # round toward zero instead of nearest-even
        a = np.asarray(x, np.float32).astype(np.float64)
        vals = O.fp8_e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
        idx = np.searchsorted(vals, np.abs(a), side="right") - 1
        return (np.clip(idx, 0, 0x7E) | np.where(np.signbit(a), 0x80, 0)).astype(np.uint8)

    def dec_bias8(c):                               # exponent bias 8 (the fnuz variant)
        return real_dec(c) / 2.0

    def q_qmax_wrong(x, mode):                      # int8 step of 128 instead of 127
        saved = dict(O.PTH_QMAX)
        O.PTH_QMAX["int8"] = 128.0
        try:
            return real_q(x, mode)
        finally:
            O.PTH_QMAX.clear()
            O.PTH_QMAX.update(saved)

    def attn_no_scale(*args, **kw):                 # softmax_scale dropped
        args = list(args)
        args[8] = 1.0
        return real_attn(*args, **kw)

    real_attn = O.pth_paged_attention
    for name, fake in (("fp8_e4m3fn_encode", enc_truncating), ("fp8_e4m3fn_decode", dec_bias8),
                       ("quantize_pth", q_qmax_wrong), ("pth_paged_attention", attn_no_scale)):
        with monkeypatch.context() as m:
            m.setattr(O, name, fake)
            assert not _pth_pins_pass(), f"planted mistake in {name} not caught"
    assert _pth_pins_pass()
