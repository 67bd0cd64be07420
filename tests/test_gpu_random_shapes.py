"""Seeded random shapes through the whole int4 path: head size, group, page
size, query lengths (decode, multi-token, prefill chunks, empty), context
lengths and work schedule are drawn per case, so that combinations no
hand-written case lists (row blocks with ragged groups, stream-K pieces over
short sequences, merges over few or many pieces) meet the oracle.

Gates: codes and scales bit-exact (G1), attention atol = rtol = 1e-2 against
the fp64 oracle reading the GPU-written cache (G2).
"""
import numpy as np
import pytest

from gpu_helpers import W, run_gpu
from test_gpu_attention import _g1, _g2

pytestmark = pytest.mark.gpu

SCHEDULES = [
    {},
    {"KV4_FORCE_PATH": "mfma"},
    {"KV4_FORCE_PATH": "mfma", "KV4_SK_GRID": "5"},
    {"KV4_FORCE_PATH": "mfma", "KV4_STREAMK": "0", "KV4_SPLIT_TOKENS": "96"},
    {"KV4_FORCE_PATH": "mfma", "KV4_REDUCE_ROWS": "1"},
    {"KV4_FORCE_PATH": "mfma", "KV4_FUSED_PLAN": "0"},
    {"KV4_FORCE_PATH": "mfma", "KV4_MFMA_RB": "1"},
    {"KV4_FORCE_PATH": "valu"},
]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    hs = int(rng.choice([64, 96, 128, 192, 80]))
    nkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 24]))
    bs = int(rng.choice([16, 32, 16, 8]))
    nseq = int(rng.integers(1, 7))
    kind = rng.choice(["decode", "multi", "prefill", "mixed"])
    ql, sl = [], []
    for _ in range(nseq):
        if kind == "decode":
            q = 1
        elif kind == "multi":
            q = int(rng.integers(1, 9))
        elif kind == "prefill":
            q = int(rng.integers(1, 60))
        else:
            q = int(rng.choice([0, 1, 1, 5, 33]))
        ctx = int(rng.integers(0, 700))
        ql.append(q)
        sl.append(q + ctx)
    if sum(ql) == 0:
        ql[0], sl[0] = 1, max(sl[0], 1)
    sched = SCHEDULES[seed % len(SCHEDULES)]
    return hs, nkv, g, bs, ql, sl, sched


@pytest.mark.parametrize("seed", range(120))
def test_random_shape(seed, monkeypatch):
    hs, nkv, g, bs, ql, sl, sched = _case(seed)
    for k, v in sched.items():
        monkeypatch.setenv(k, v)
    w = W.custom(f"rand{seed}", nkv * g, nkv, hs, ql, sl, block_size=bs, seed=seed, outlier_frac=0.01)
    # every third case passes loose host-side bounds (upper bounds, not maxima)
    slack = (3, 2 * w.max_seq_len + 17) if seed % 3 == 2 else (0, 0)
    r = run_gpu(w, len_slack=slack)
    _g1(r)
    _g2(r)


@pytest.mark.parametrize("seed", range(60))
def test_random_shape_modes_layouts_windows(seed, monkeypatch):
    """The same draws through the layout entry points: int4 / int8 / fp8
    caches, packed or inline-scale rows, with or without a sliding window."""
    from test_gpu_window import _run
    hs, nkv, g, bs, ql, sl, sched = _case(500 + seed)
    for k, v in sched.items():
        monkeypatch.setenv(k, v)
    rng = np.random.default_rng(7000 + seed)
    mode = ["int4", "int8", "fp8"][seed % 3]
    inline = bool(rng.integers(0, 2))
    window = int(rng.choice([0, 0, 1, 9, 64, 300]))
    w = W.custom(f"randl{seed}", nkv * g, nkv, hs, ql, sl, block_size=bs, seed=seed, outlier_frac=0.01)
    _run(w, mode, window, inline=inline)


@pytest.mark.parametrize("seed", range(40))
def test_random_write(seed):
    """kv4_rht_write on random head sizes (any multiple of 8 up to 256),
    kv head counts, page sizes and slot maps (shuffled, repeated pages,
    negative and past-the-end slots, which are skipped), against the oracle
    bit for bit over the whole cache (untouched bytes keep the fill)."""
    from test_gpu_write import _write_and_compare
    rng = np.random.default_rng(9000 + seed)
    hs = 8 * int(rng.integers(1, 33))
    nkv = int(rng.integers(1, 9))
    bs = int(rng.choice([1, 8, 16, 32]))
    T = int(rng.integers(0, 400))
    nb = max(1, (T + bs - 1) // bs + int(rng.integers(0, 3)))
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    if T:
        bad = rng.random(T) < 0.05
        slots[bad] = rng.choice([-1, -7, nb * bs, nb * bs + 5], int(bad.sum()))
    gain = np.where(rng.random((nkv, hs)) < 0.02, 20.0, 1.0).astype(np.float32)   # a few outlier channels
    key = W.normal_bf16((T, nkv, hs), seed=seed, gain=gain)
    value = W.normal_bf16((T, nkv, hs), seed=seed + 10 ** 6)
    _write_and_compare(key, value, slots, nb, bs, seed=0x1234 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_short_sequences_and_odd_pages(seed, monkeypatch):
    """Draws in which some sequences are shorter than their query block (the
    first rows of such a sequence see no key and must come out as exactly 0,
    as the oracle returns them) and, every other case, a page size that is not
    a power of two (12 or 24 tokens, served by the vector kernel). G1 and G2
    over every row."""
    hs, nkv, g, bs, ql, sl, sched = _case(3000 + seed)
    rng = np.random.default_rng(5000 + seed)
    for i, q in enumerate(ql):
        if q > 1 and rng.random() < 0.6:
            sl[i] = int(rng.integers(0, q))
    if seed % 2:
        bs = int(rng.choice([12, 24]))
    for k, v in sched.items():
        monkeypatch.setenv(k, v)
    w = W.custom(f"rshort{seed}", nkv * g, nkv, hs, ql, sl, block_size=bs, seed=seed, outlier_frac=0.01)
    r = run_gpu(w)
    _g1(r)
    got, ref = _g2(r)
    qsl = r.lay.query_start_loc
    for s, (q, L) in enumerate(zip(ql, sl)):
        if q > L:
            rows = slice(int(qsl[s]), int(qsl[s]) + q - L)
            assert not got[rows].any() and not ref[rows].any()
