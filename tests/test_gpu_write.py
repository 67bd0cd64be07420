"""Write path parity: codes and scales from kv4_rht_write are bit-exact
against the oracle's spec tier on the same seeded inputs."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, alloc_cache, host, kv4, say

pytestmark = pytest.mark.gpu


def _write_and_compare(key_bf16, value_bf16, slots, num_blocks, bs, seed, fill=0xA5, key_dev=None,
                       value_dev=None):
    T, nkv, hs = key_bf16.shape
    w = W.custom("w", nkv, nkv, hs, [1], [1], block_size=bs)
    kc, vc, ks, vs = alloc_cache(w, num_blocks, fill)
    kd = key_bf16.to(DEV) if key_dev is None else key_dev
    vd = value_bf16.to(DEV) if value_dev is None else value_dev
    kv4.kv4_rht_write(kd, vd, kc, vc, ks, vs, torch.from_numpy(slots).to(DEV), sign_seed=seed)
    torch.cuda.synchronize()
    key, value = key_bf16.float().numpy(), value_bf16.float().numpy()
    okc, oks = O.new_cache(num_blocks, bs, nkv, hs)
    ovc, ovs = O.new_cache(num_blocks, bs, nkv, hs)
    okc[:] = fill
    ovc[:] = fill
    oks[:] = float(fill)
    ovs[:] = float(fill)
    O.rht_write(key, okc, oks, slots, seed)
    O.rht_write(value, ovc, ovs, slots, seed)
    np.testing.assert_array_equal(host(kc), okc)
    np.testing.assert_array_equal(host(vc), ovc)
    np.testing.assert_array_equal(host(ks).view(np.uint32), oks.view(np.uint32))
    np.testing.assert_array_equal(host(vs).view(np.uint32), ovs.view(np.uint32))


@pytest.mark.parametrize("hs", [8, 16, 24, 64, 80, 96, 120, 128, 136, 192, 256])
def test_write_bit_exact_head_sizes(hs):
    say(f"[gpu] write hs={hs}")
    T, nkv, bs = 300, 3, 16
    key = W.normal_bf16((T, nkv, hs), seed=hs)
    value = W.normal_bf16((T, nkv, hs), seed=hs + 1000)
    nb = (T + bs - 1) // bs + 3
    slots = np.random.default_rng(hs).permutation(nb * bs)[:T].astype(np.int64)
    _write_and_compare(key, value, slots, nb, bs, seed=42)


@pytest.mark.parametrize("bs,nkv,seed", [(1, 1, 0), (8, 8, 7), (32, 2, 123456789), (16, 32, 2 ** 63 + 5)])
def test_write_bit_exact_layouts(bs, nkv, seed):
    say(f"[gpu] write bs={bs} nkv={nkv} seed={seed}")
    T, hs = 257, 128
    key = W.normal_bf16((T, nkv, hs), seed=bs)
    value = W.normal_bf16((T, nkv, hs), seed=bs + 1)
    nb = (T + bs - 1) // bs + 1
    slots = np.random.default_rng(bs).permutation(nb * bs)[:T].astype(np.int64)
    _write_and_compare(key, value, slots, nb, bs, seed=seed)


def test_write_skips_invalid_slots_and_strided_rows():
    say("[gpu] write skip + strided")
    T, nkv, hs, bs = 100, 4, 96, 16
    big = W.normal_bf16((T, 3 * nkv, hs), seed=5)       # e.g. a fused qkv buffer
    key_dev, value_dev = big.to(DEV)[:, :nkv], big.to(DEV)[:, nkv:2 * nkv]
    key, value = big[:, :nkv].contiguous(), big[:, nkv:2 * nkv].contiguous()
    nb = 10
    slots = np.random.default_rng(1).permutation(nb * bs)[:T].astype(np.int64)
    slots[::7] = -1
    slots[3] = nb * bs          # one past the end: skipped
    slots[11] = 10 ** 12
    _write_and_compare(key, value, slots, nb, bs, seed=42, key_dev=key_dev, value_dev=value_dev)


def test_write_zero_outlier_and_extreme_vectors():
    say("[gpu] write zeros / outliers / extremes")
    T, nkv, hs, bs = 64, 2, 128, 16
    x = W.normal_bf16((T, nkv, hs), seed=9).float()
    x[0] = 0.0                                   # amax == 0 -> scale 0, codes 0
    x[1, 0, 5] = 1e4                             # a single outlier channel
    x[2] *= 1e30                                 # large, finite after rotation
    x[3] *= 1e-30
    x[4] *= 1e-37                                # scales in the float32 subnormal range
    x[5, 1] = 0.0
    x[6] = torch.sign(x[6]) * 2.0 ** -133        # bf16 subnormals
    key = x.to(torch.bfloat16)
    value = (-x).to(torch.bfloat16)
    slots = np.arange(T, dtype=np.int64)
    _write_and_compare(key, value, slots, T // bs, bs, seed=42)


@pytest.mark.parametrize("hs", [128, 96])
def test_write_exact_ties(hs):
    """Vectors whose rotated values are 7 * 2^k on one element and half-integer
    multiples of 2^k on three others (inputs from the oracle's exact inverse
    rotation, exact in bf16): scale = 2^k exactly, so every nonzero quotient
    y / scale is a whole or half integer and the codes of the halves are
    decided by ties to even, for K and for -K (the negated vectors)."""
    say(f"[gpu] write exact ties hs={hs}")
    T, nkv, bs, seed = 48, 2, 16, 42
    rng = np.random.default_rng(17 + hs)
    y = np.zeros((T, nkv, hs))
    for t in range(T):
        for h in range(nkv):
            idx = rng.choice(hs, 4, replace=False)
            y[t, h, idx[0]] = 7.0 * rng.choice([-1.0, 1.0])
            y[t, h, idx[1:]] = rng.integers(-14, 15, 3) / 2.0
            y[t, h] *= 2.0 ** int(rng.integers(-20, 21))
    x = O.unrotate_math(y, O.rht_signs(seed, hs)).astype(np.float32)
    assert np.array_equal(O.bf16_round(x), x)             # exact inputs
    yr = O.rotate_spec(x, O.rht_signs(seed, hs))
    assert np.array_equal(yr, y.astype(np.float32))       # the rotation lands on y exactly
    _, scale = O.quantize_int4(yr)
    q = yr / scale[..., None]
    assert (np.abs(q - np.floor(q)) == 0.5).sum() > T      # exact ties are present
    key = torch.from_numpy(x).to(torch.bfloat16)
    value = (-key.float()).to(torch.bfloat16)
    slots = np.random.default_rng(5).permutation(T).astype(np.int64)
    _write_and_compare(key, value, slots, T // bs, bs, seed=seed)


def test_write_many_tokens():
    say("[gpu] write 40000 tokens")
    T, nkv, hs, bs = 40000, 8, 64, 16
    key = W.normal_bf16((T, nkv, hs), seed=77)
    value = W.normal_bf16((T, nkv, hs), seed=78)
    nb = T // bs + 5
    slots = np.random.default_rng(3).permutation(nb * bs)[:T].astype(np.int64)
    _write_and_compare(key, value, slots, nb, bs, seed=1)


def test_write_empty_is_noop():
    w = W.custom("w", 2, 2, 64, [1], [1])
    kc, vc, ks, vs = alloc_cache(w, 2, 7)
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    kv4.kv4_rht_write(e, e, kc, vc, ks, vs, torch.empty(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert int(kc.min()) == 7 and int(kc.max()) == 7


@pytest.mark.parametrize("hs", [96, 128, 192])
def test_dequant_matches_oracle(hs):
    say(f"[gpu] dequant hs={hs}")
    T, nkv, bs = 200, 2, 16
    key = W.normal_bf16((T, nkv, hs), seed=hs + 3)
    nb = (T + bs - 1) // bs
    slots = np.arange(T, dtype=np.int64)
    w = W.custom("w", nkv, nkv, hs, [1], [1], block_size=bs)
    kc, vc, ks, vs = alloc_cache(w, nb)
    kv4.kv4_rht_write(key.to(DEV), key.to(DEV), kc, vc, ks, vs, torch.from_numpy(slots).to(DEV))
    sl = torch.from_numpy(np.concatenate([slots[::3], [-1, nb * bs]])).to(DEV)
    raw = host(kv4.kv4_dequant(kc, ks, sl, inverse_rotate=False))
    back = host(kv4.kv4_dequant(kc, ks, sl, inverse_rotate=True))
    torch.cuda.synchronize()
    s_np = host(sl)
    ok = s_np[:-2]
    want_raw = O.dequant(host(kc), host(ks), ok, 42, inverse_rotate=False)
    np.testing.assert_array_equal(raw[:-2].view(np.uint32), want_raw.view(np.uint32))
    assert not raw[-2:].any() and not back[-2:].any()          # out-of-range slots -> zeros
    want_back = O.dequant(host(kc), host(ks), ok, 42, inverse_rotate=True)
    np.testing.assert_allclose(back[:-2], want_back, rtol=0, atol=1e-5 * np.abs(want_back).max())
    # the round trip itself (pages: int4 deq_atol = deq_rtol = 0.5)
    x = key.float().numpy()[::3]
    bad = np.abs(back[:-2] - x) > 0.5 + 0.5 * np.abs(x)
    assert bad.mean() < 1e-3


def test_duplicate_slots_debug_check(monkeypatch):
    """KV4_CHECK_SLOTS=1: a slot map that names one slot twice is rejected
    before any launch (the cache keeps its fill); without the variable the
    call runs (duplicates race, by contract); a map without duplicates passes
    the check and is written bit-exactly."""
    T, nkv, hs, bs, nb = 40, 2, 64, 16, 4
    key = W.normal_bf16((T, nkv, hs), seed=5)
    value = W.normal_bf16((T, nkv, hs), seed=6)
    dup = np.arange(T, dtype=np.int64)
    dup[17] = dup[3]
    dup[20] = -1                      # skipped slots are not duplicates
    dup[21] = -1
    w = W.custom("dup", nkv, nkv, hs, [1], [1], block_size=bs)
    kc, vc, ks, vs = alloc_cache(w, nb, 0xA5)
    monkeypatch.setenv("KV4_CHECK_SLOTS", "1")
    with pytest.raises(kv4.Kv4Error, match="slot 3 appears at tokens 3 and 17"):
        kv4.kv4_rht_write(key.to(DEV), value.to(DEV), kc, vc, ks, vs, torch.from_numpy(dup).to(DEV), sign_seed=1)
    torch.cuda.synchronize()
    assert (host(kc) == 0xA5).all() and (host(vc) == 0xA5).all()
    uniq = np.random.default_rng(0).permutation(nb * bs)[:T].astype(np.int64)
    uniq[5] = -1
    _write_and_compare(key, value, uniq, nb, bs, seed=1)
    monkeypatch.delenv("KV4_CHECK_SLOTS")
    kv4.kv4_rht_write(key.to(DEV), value.to(DEV), kc, vc, ks, vs, torch.from_numpy(dup).to(DEV), sign_seed=1)
    torch.cuda.synchronize()
