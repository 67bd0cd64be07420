"""Host-side helpers of the GPU tests, checked on the CPU."""
import numpy as np
import pytest

from gpu_helpers import O, inline_rows


@pytest.mark.parametrize("mode,nkv,hs,bs", [("int4", 2, 96, 4), ("int8", 3, 64, 2), ("fp8", 1, 128, 3)])
def test_inline_rows_matches_oracle_unpack(mode, nkv, hs, bs):
    rng = np.random.default_rng(hs + nkv)
    geo = O.inline_geometry(mode, nkv, hs, bs)
    nb = 5
    buf = rng.integers(0, 256, size=(nb, geo["block_bytes"]), dtype=np.uint8)
    want = O.inline_unpack(buf, mode, nkv, hs, bs)
    got = inline_rows(buf, mode, nkv, hs, bs)
    for a, b in zip(got[:2], want[:2]):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(got[2:4], want[2:4]):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    # the padding bytes are exactly those inline_pack leaves zero
    zeroed = O.inline_pack(*want, mode)
    assert not inline_rows(zeroed, mode, nkv, hs, bs)[4].any()
    assert got[4].shape[-1] == geo["pitch"] - geo["code_bytes"] - 4
