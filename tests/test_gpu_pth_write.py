"""Write path parity of the per-token-head INT8 / FP8 control modes: codes
and scales from kv4_pth_write are bit-exact against the oracle on the same
seeded inputs; kv4_pth_dequant matches the oracle's float32 products."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, host, kv4, say

pytestmark = pytest.mark.gpu

MODES = ["int8", "fp8"]


def _alloc(nb, bs, nkv, hs, fill):
    kc = torch.full((nb, bs, nkv, hs), fill, dtype=torch.uint8, device=DEV)
    ks = torch.full((nb, bs, nkv), float(fill), dtype=torch.float32, device=DEV)
    return kc, torch.full_like(kc, fill), ks, torch.full_like(ks, float(fill))


def _write_and_compare(mode, key_bf16, value_bf16, slots, nb, bs, fill=0xA5, key_dev=None, value_dev=None):
    T, nkv, hs = key_bf16.shape
    kc, vc, ks, vs = _alloc(nb, bs, nkv, hs, fill)
    kd = key_bf16.to(DEV) if key_dev is None else key_dev
    vd = value_bf16.to(DEV) if value_dev is None else value_dev
    kv4.kv4_pth_write(mode, kd, vd, kc, vc, ks, vs, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    key, value = key_bf16.float().numpy(), value_bf16.float().numpy()
    okc, oks = O.pth_new_cache(nb, bs, nkv, hs)
    ovc, ovs = O.pth_new_cache(nb, bs, nkv, hs)
    for c in (okc, ovc):
        c[:] = fill
    for c in (oks, ovs):
        c[:] = float(fill)
    O.pth_write(key, okc, oks, slots, mode)
    O.pth_write(value, ovc, ovs, slots, mode)
    np.testing.assert_array_equal(host(kc), okc)
    np.testing.assert_array_equal(host(vc), ovc)
    np.testing.assert_array_equal(host(ks).view(np.uint32), oks.view(np.uint32))
    np.testing.assert_array_equal(host(vs).view(np.uint32), ovs.view(np.uint32))
    return kc, ks


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("hs", [8, 24, 64, 96, 128, 192, 256])
def test_pth_write_bit_exact_head_sizes(mode, hs):
    say(f"[gpu] pth write {mode} hs={hs}")
    T, nkv, bs = 300, 3, 16
    key = W.normal_bf16((T, nkv, hs), seed=hs)
    value = W.normal_bf16((T, nkv, hs), seed=hs + 1000)
    nb = (T + bs - 1) // bs + 3
    slots = np.random.default_rng(hs).permutation(nb * bs)[:T].astype(np.int64)
    _write_and_compare(mode, key, value, slots, nb, bs)


@pytest.mark.parametrize("mode", MODES)
def test_pth_write_skips_invalid_slots_and_strided_rows(mode):
    say(f"[gpu] pth write {mode} skip + strided")
    T, nkv, hs, bs = 100, 4, 128, 16
    big = W.normal_bf16((T, 3 * nkv, hs), seed=5)
    key_dev, value_dev = big.to(DEV)[:, :nkv], big.to(DEV)[:, nkv:2 * nkv]
    key, value = big[:, :nkv].contiguous(), big[:, nkv:2 * nkv].contiguous()
    nb = 10
    slots = np.random.default_rng(1).permutation(nb * bs)[:T].astype(np.int64)
    slots[::7] = -1
    slots[3] = nb * bs
    slots[11] = 10 ** 12
    _write_and_compare(mode, key, value, slots, nb, bs, key_dev=key_dev, value_dev=value_dev)


@pytest.mark.parametrize("mode", MODES)
def test_pth_write_zero_outlier_and_extreme_vectors(mode):
    say(f"[gpu] pth write {mode} zeros / outliers / extremes")
    T, nkv, hs, bs = 64, 2, 128, 16
    x = W.normal_bf16((T, nkv, hs), seed=9).float()
    x[0] = 0.0                                   # amax == 0 -> scale 0, codes 0
    x[1, 0, 5] = 1e4                             # one outlier: most codes round to 0 / subnormal fp8
    x[2] *= 1e30
    x[3] *= 1e-30
    x[4] *= 1e-37                                # scales in the float32 subnormal range
    x[5, :, ::2] = -0.0                          # negative zeros
    x[6, 1] = torch.linspace(-1.0, 1.0, hs)      # exact ties of the int8 / fp8 grids
    key = x.to(torch.bfloat16)
    value = (x * -0.5).to(torch.bfloat16)
    slots = np.arange(T, dtype=np.int64)
    _write_and_compare(mode, key, value, slots, T // bs, bs)


@pytest.mark.parametrize("mode", MODES)
def test_pth_dequant_matches_oracle(mode):
    say(f"[gpu] pth dequant {mode}")
    T, nkv, hs, bs = 200, 2, 64, 16
    key = W.normal_bf16((T, nkv, hs), seed=3)
    nb = (T + bs - 1) // bs + 1
    slots = np.random.default_rng(2).permutation(nb * bs)[:T].astype(np.int64)
    kc, ks = _write_and_compare(mode, key, key, slots, nb, bs, fill=0)
    q = slots.copy()
    q[5] = -1                                    # out-of-range slots give zeros
    got = host(kv4.kv4_pth_dequant(mode, kc, ks, torch.from_numpy(q).to(DEV)))
    ref = O.pth_dequant(host(kc), host(ks), np.where(q < 0, 0, q), mode)
    ref[5] = 0.0
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
