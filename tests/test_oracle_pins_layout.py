"""Pins of the oracle's inline-scale padded-slot layout against the float32
views the pages give for it (vLLM PR #40835 review of `_ensure_scale_caches`:
full_block_f32, slot_f32, head_f32, scale_off_f32, V scales kv_half_bytes
after K) and the 16-byte row alignment of vLLM PR #62113. The views are
written out here from the page formulas; the oracle computes byte offsets
its own way, so a wrong offset, order or padding shows up as a mismatch."""
import numpy as np
import pytest

from oracle import kv4_oracle as O

MODES = ["int4", "int8", "fp8"]


def _random_caches(mode, nb, bs, nkv, hs, seed=0):
    rng = np.random.default_rng(seed)
    c = hs // 2 if mode == "int4" else hs
    kc = rng.integers(0, 256, (nb, bs, nkv, c), dtype=np.uint8)
    vc = rng.integers(0, 256, (nb, bs, nkv, c), dtype=np.uint8)
    ks = (rng.standard_normal((nb, bs, nkv)) * 10).astype(np.float32)
    vs = (rng.standard_normal((nb, bs, nkv)) * 10).astype(np.float32)
    ks[0, 0, 0] = -0.0
    vs[-1, -1, -1] = np.float32(1e-40)                # subnormal
    return kc, vc, ks, vs


def _page_views(mode, nkv, hs, bs):
    """The page formulas with dtype_sz = 1 (uint8 cache), padded_hs * dtype_sz
    the 16-byte-rounded row of codes + one float32 scale."""
    c = hs // 2 if mode == "int4" else hs
    padded = ((c + 4 + 15) // 16) * 16
    kv_half_bytes = bs * nkv * padded
    return dict(full_block_f32=2 * kv_half_bytes // 4, slot_f32=nkv * padded // 4, head_f32=padded // 4,
                scale_off_f32=c // 4, kv_half_f32=kv_half_bytes // 4, c=c, padded=padded)


def test_inline_geometry_worked_examples():
    # hand-derived: int4 hs 128 -> 64 code bytes + 4 -> pitch 80; 2 heads x 16 slots x 80 = 2560 per half
    g = O.inline_geometry("int4", 2, 128, 16)
    assert (g["code_bytes"], g["pitch"], g["kv_half_bytes"], g["block_bytes"]) == (64, 80, 2560, 5120)
    assert (g["full_block_f32"], g["slot_f32"], g["head_f32"], g["scale_off_f32"]) == (1280, 40, 20, 16)
    # int8 hs 96: 96 + 4 -> 112; 4 heads x 16 slots x 112 = 7168 per half
    g = O.inline_geometry("int8", 4, 96, 16)
    assert (g["pitch"], g["kv_half_bytes"], g["full_block_f32"], g["slot_f32"], g["head_f32"],
            g["scale_off_f32"]) == (112, 7168, 3584, 112, 28, 24)
    # int4 hs 8: 4 code bytes + 4 -> one 16-byte row
    g = O.inline_geometry("int4", 1, 8, 1)
    assert (g["pitch"], g["block_bytes"]) == (16, 32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("nkv,hs,bs", [(2, 128, 16), (3, 96, 8), (1, 64, 1), (4, 8, 4)])
def test_inline_scales_sit_at_the_pages_float32_views(mode, nkv, hs, bs):
    nb = 3
    kc, vc, ks, vs = _random_caches(mode, nb, bs, nkv, hs)
    buf = O.inline_pack(kc, vc, ks, vs, mode)
    v = _page_views(mode, nkv, hs, bs)
    f32 = buf.reshape(-1).view(np.uint32)          # bit patterns, so -0.0 and subnormals compare exactly
    for p in range(nb):
        for t in range(bs):
            for h in range(nkv):
                i = p * v["full_block_f32"] + t * v["slot_f32"] + h * v["head_f32"] + v["scale_off_f32"]
                assert f32[i] == ks[p, t, h].view(np.uint32)
                assert f32[i + v["kv_half_f32"]] == vs[p, t, h].view(np.uint32)


@pytest.mark.parametrize("mode", MODES)
def test_inline_codes_padding_and_16_byte_rows(mode):
    nb, bs, nkv, hs = 2, 4, 3, 96
    kc, vc, ks, vs = _random_caches(mode, nb, bs, nkv, hs, seed=1)
    buf = O.inline_pack(kc, vc, ks, vs, mode).reshape(-1)
    v = _page_views(mode, nkv, hs, bs)
    c, padded = v["c"], v["padded"]
    assert padded % 16 == 0 and buf.size == nb * 4 * v["full_block_f32"]
    for p in range(nb):
        for half, codes in enumerate((kc, vc)):
            for t in range(bs):
                for h in range(nkv):
                    start = 4 * (p * v["full_block_f32"] + half * v["kv_half_f32"] + t * v["slot_f32"] +
                                 h * v["head_f32"])
                    assert start % 16 == 0
                    assert np.array_equal(buf[start:start + c], codes[p, t, h])
                    assert not buf[start + c + 4:start + padded].any()


@pytest.mark.parametrize("mode", MODES)
def test_inline_roundtrip(mode):
    kc, vc, ks, vs = _random_caches(mode, 4, 16, 2, 128, seed=2)
    out = O.inline_unpack(O.inline_pack(kc, vc, ks, vs, mode), mode, 2, 128, 16)
    for a, b in zip(out, (kc, vc, ks, vs)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_inline_store_rows_touches_only_the_written_slots():
    mode, nb, bs, nkv, hs = "int4", 3, 4, 2, 64
    kc, vc, ks, vs = _random_caches(mode, nb, bs, nkv, hs, seed=3)
    geo = O.inline_geometry(mode, nkv, hs, bs)
    buf = np.full((nb, geo["block_bytes"]), 0xA5, dtype=np.uint8)
    slots = np.array([5, 0, 11, -1, nb * bs], dtype=np.int64)
    O.inline_store_rows(buf, kc, vc, ks, vs, slots, mode)
    full = O.inline_pack(kc, vc, ks, vs, mode).reshape(-1)
    flat = buf.reshape(-1)
    written = np.zeros(flat.size, dtype=bool)
    for s in (5, 0, 11):
        p, t = s // bs, s % bs
        for half in (0, 1):
            for h in range(nkv):
                o = O.inline_row_offset(geo, p, half, t, h, nkv)
                written[o:o + geo["code_bytes"] + 4] = True
    assert np.array_equal(flat[written], full[written])
    assert (flat[~written] == 0xA5).all()


def test_planted_layout_mistakes_are_caught(monkeypatch):
    real = O.inline_geometry

    def v_not_offset(mode, nkv, hs, bs):           # V rows on top of K rows
        g = dict(real(mode, nkv, hs, bs))
        g["kv_half_bytes"] = 0
        return g

    def pitch_unaligned(mode, nkv, hs, bs):        # rows not padded to 16 bytes
        g = dict(real(mode, nkv, hs, bs))
        c = g["code_bytes"]
        g["pitch"] = c + 4
        g["kv_half_bytes"] = bs * nkv * (c + 4)
        g["block_bytes"] = 2 * g["kv_half_bytes"]
        return g

    def scale_first(geo, page, half, slot, head, nkv):   # rows shifted by one scale
        return real_off(geo, page, half, slot, head, nkv) + 4

    real_off = O.inline_row_offset
    for name, fake in (("inline_geometry", v_not_offset), ("inline_geometry", pitch_unaligned),
                       ("inline_row_offset", scale_first)):
        with monkeypatch.context() as m:
            m.setattr(O, name, fake)
            with pytest.raises((AssertionError, ValueError, IndexError)):
                test_inline_scales_sit_at_the_pages_float32_views("int4", 2, 128, 16)
                test_inline_codes_padding_and_16_byte_rows("int8")
