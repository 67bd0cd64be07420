"""Parity at the full sizes of every benchmark workload, in the launch
configuration bench.py times: every KV token written in one write call, one
attention call over the whole batch (workspace sized by the library).

Workloads: Phi-3 (hs 96), Llama-3.2-1B (GQA 4, hs 64), Qwen2.5-1.5B mixed
chunked prefill + decode and its prefill chunks alone, Llama-3-8B long
context (hs 128, x20 outlier channels) with its head-size-192 sweep, its
multi-token decode and a head-size-256 GQA variant (16 / 4 heads), and the
Llama-3-8B shape again with the int8 and fp8 control caches, a 4096-token
sliding window and the inline-scale padded-slot layout.

Gates, over everything the call produced (no sampling):
  * G1 -- every written token's codes and scale bit-exact against the
    oracle's spec tier, streamed from the device in chunks of token rows and
    checked on a pool of CPU workers;
  * G2 -- every query row within atol = rtol = 1e-2 of the fp64 oracle
    reading the GPU-written cache;
  * G4 -- every query row against unquantized fp64 attention on the same bf16
    inputs at the pages' atol = rtol = 5e-2 (vLLM PR #62881, Tolerance). The
    max abs error and the correlation are printed for the GPU and for the
    oracle's own quantized result. The bound is asserted on every row where
    the oracle's quantized result meets it with a quarter of it to spare: on
    rows where the method itself misses it (the x20 outlier channels make
    the logits so peaked that int4 noise in K moves the softmax mass), no
    implementation of the method can meet it.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, host, inline_rows, kv4, say, worker_count

pytestmark = pytest.mark.gpu

G2_TOL = 1e-2
G4_TOL = 5e-2
G4_ASSERT_SLACK = 0.75     # rows whose oracle error uses at most this share of the G4 bound
G1_CHUNK = 16384           # token rows per G1 job

# id -> (workload, cache mode, sliding window, inline-scale layout)
CASES = {
    "phi3": ("phi3", "int4", 0, False),
    "llama1b": ("llama1b", "int4", 0, False),
    "qwen_mixed": ("qwen_mixed", "int4", 0, False),
    "qwen_prefill": ("qwen_prefill", "int4", 0, False),
    "llama8b_long": ("llama8b_long", "int4", 0, False),
    "llama8b_hs192": ("llama8b_hs192", "int4", 0, False),
    "hs256_long": ("hs256_long", "int4", 0, False),
    "llama8b_spec": ("llama8b_spec", "int4", 0, False),
    "llama8b_long_int8": ("llama8b_long", "int8", 0, False),
    "llama8b_long_fp8": ("llama8b_long", "fp8", 0, False),
    "llama8b_long_window4096": ("llama8b_long", "int4", 4096, False),
    "llama8b_long_inline": ("llama8b_long", "int4", 0, True),
}


@dataclasses.dataclass
class FullRun:
    w: W.Workload
    lay: W.Layout
    mode: str
    window: int
    inline: bool
    key: torch.Tensor          # bf16 [T, nkv, hs] on the device
    value: torch.Tensor
    query: torch.Tensor        # bf16 [Tq, nq, hs] on the device
    slots: np.ndarray          # slot of every KV token row
    packed: tuple | None       # (kc, vc, ks, vs) device tensors of the packed layout
    lcache: object | None      # kv4.LayoutCache of the inline layout
    out: torch.Tensor

    @property
    def code_bytes(self) -> int:
        return self.w.head_size // 2 if self.mode == "int4" else self.w.head_size


def _full_run(cfg: str, mode: str, window: int, inline: bool) -> FullRun:
    w = W.ALL[cfg]()
    lay = W.make_layout(w)
    say(f"[gpu] full size {w.name} mode={mode} window={window} inline={inline}: seqs={w.num_seqs} "
        f"kv_tokens={w.total_kv_tokens} q_tokens={w.num_q_tokens}")
    t = W.make_tensors(w, lay, device=DEV)
    slots = W.all_slots(lay, w)
    sl = torch.from_numpy(slots).to(DEV)
    nb, bs, nkv, hs = lay.num_blocks, w.block_size, w.num_kv_heads, w.head_size
    bt = torch.from_numpy(lay.block_table).to(DEV)
    slens = torch.from_numpy(lay.seq_lens).to(DEV)
    qsl = torch.from_numpy(lay.query_start_loc).to(DEV)
    packed, lcache = None, None
    if inline:
        lcache = kv4.LayoutCache.inline(mode, nb, bs, nkv, hs, device=DEV)
    else:
        c = hs // 2 if mode == "int4" else hs
        kc = torch.zeros((nb, bs, nkv, c), dtype=torch.uint8, device=DEV)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb, bs, nkv), dtype=torch.float32, device=DEV)
        vs = torch.zeros_like(ks)
        packed = (kc, vc, ks, vs)
        if window:
            lcache = kv4.packed_layout_cache(mode, kc, vc, ks, vs)
    # the entry points bench.py uses for this variant
    if lcache is not None:
        kv4.kv4_write_layout(t.key, t.value, lcache, sl, sign_seed=w.sign_seed)
        out = kv4.kv4_attention_layout(t.query, lcache, bt, slens, qsl, w.max_query_len, w.max_seq_len,
                                       sign_seed=w.sign_seed, sliding_window=window)
    elif mode == "int4":
        kv4.kv4_rht_write(t.key, t.value, *packed, sl, sign_seed=w.sign_seed)
        out = kv4.kv4_paged_attention(t.query, *packed, bt, slens, qsl, max_query_len=w.max_query_len,
                                      max_seq_len=w.max_seq_len, sign_seed=w.sign_seed)
    else:
        kv4.kv4_pth_write(mode, t.key, t.value, *packed, sl)
        out = kv4.kv4_pth_attention(mode, t.query, *packed, bt, slens, qsl, max_query_len=w.max_query_len,
                                    max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    return FullRun(w, lay, mode, window, inline, t.key, t.value, t.query, slots, packed, lcache, out)


@pytest.fixture(scope="module", params=list(CASES), ids=list(CASES))
def full(request):
    run = _full_run(*CASES[request.param])
    yield run
    del run
    torch.cuda.empty_cache()


def _pool():
    from threadpoolctl import threadpool_limits
    return cf.ThreadPoolExecutor(max_workers=worker_count()), threadpool_limits(limits=1)


def _drain(futs, results, keep: int):
    while len(futs) > keep:
        results.append(futs.pop(0).result())


# ------------------------------------------------------------------ G1

def _rows_of_slots(run: FullRun, which: int, slots: np.ndarray):
    """Codes [n, nkv, C] and scales [n, nkv] stored at `slots` in the K
    (which = 0) or V (1) cache, copied to the host; for the inline layout also
    the rows' padding bytes."""
    w = run.w
    nkv, bs, c = w.num_kv_heads, w.block_size, run.code_bytes
    st = torch.from_numpy(slots).to(DEV)
    if run.inline:
        geo = O.inline_geometry(run.mode, nkv, w.head_size, bs)
        rows = run.lcache.buffer.view(run.lay.num_blocks, 2, bs, nkv, geo["pitch"])
        sel = host(rows[st // bs, which, st % bs])                          # [n, nkv, pitch]
        scales = np.ascontiguousarray(sel[..., c:c + 4]).view(np.float32)[..., 0]
        return np.ascontiguousarray(sel[..., :c]), scales, sel[..., c + 4:]
    codes_t, scale_t = run.packed[which], run.packed[2 + which]
    codes = host(codes_t.view(-1, nkv, c).index_select(0, st))
    scales = host(scale_t.view(-1, nkv).index_select(0, st))
    return codes, scales, None


def _g1_job(mode: str, signs, x: np.ndarray, codes: np.ndarray, scales: np.ndarray, pad, t0: int):
    if mode == "int4":
        qc, qs = O.quantize_int4(O.rotate_spec(x, signs))
        want = O.pack_int4(qc)
    else:
        want, qs = O.quantize_pth(x, mode)
    bad = (want != codes).any(axis=-1) | (qs.view(np.uint32) != scales.view(np.uint32))
    pad_bad = int(np.count_nonzero(pad)) if pad is not None else 0
    idx = np.argwhere(bad)
    return int(bad.sum()), (t0 + int(idx[0][0]), int(idx[0][1])) if idx.size else None, pad_bad


def test_full_size_write_bit_exact(full: FullRun):
    """G1 on every written (token, kv head) of K and of V."""
    w = full.w
    T = full.slots.shape[0]
    signs = O.rht_signs(w.sign_seed, w.head_size)
    pool, limit = _pool()
    futs, results = [], []
    with pool, limit:
        for t0 in range(0, T, G1_CHUNK):
            t1 = min(T, t0 + G1_CHUNK)
            sl = full.slots[t0:t1]
            for which, src in ((0, full.key), (1, full.value)):
                x = W.bf16_as_f32_numpy(src[t0:t1])
                codes, scales, pad = _rows_of_slots(full, which, sl)
                futs.append(pool.submit(_g1_job, full.mode, signs, x, codes, scales, pad, t0))
            _drain(futs, results, 2 * worker_count())
        _drain(futs, results, 0)
    nbad = sum(r[0] for r in results)
    first = next((r[1] for r in results if r[1] is not None), None)
    pad_bad = sum(r[2] for r in results)
    say(f"    G1: {T} tokens x {w.num_kv_heads} kv heads x (K, V) checked; mismatching vectors {nbad}"
        + (f" (first at token {first[0]}, head {first[1]})" if first else "")
        + (f"; nonzero padding bytes {pad_bad}" if full.inline else ""))
    assert nbad == 0 and pad_bad == 0


# ------------------------------------------------------------- G2 / G4

def _seq_pages(run: FullRun, s: int):
    """The sequence's pages of the GPU-written caches on the host, renumbered
    0..n-1, and a page table naming them."""
    w = run.w
    n = -(-int(w.seq_lens[s]) // w.block_size)
    pages = torch.from_numpy(run.lay.block_table[s, :n].astype(np.int64)).to(DEV)
    if run.inline:
        kc, vc, ks, vs, _ = inline_rows(host(run.lcache.buffer.index_select(0, pages)), run.mode,
                                        w.num_kv_heads, w.head_size, w.block_size)
    else:
        kc, vc, ks, vs = (host(x.index_select(0, pages)) for x in run.packed)
    bt = np.zeros_like(run.lay.block_table)
    bt[s, :n] = np.arange(n)
    return kc, vc, ks, vs, bt


def _attn_job(run: FullRun, s: int, q: np.ndarray, caches, k_raw, v_raw):
    w, lay = run.w, run.lay
    kc, vc, ks, vs, bt = caches
    q0, q1 = int(lay.query_start_loc[s]), int(lay.query_start_loc[s + 1])
    scale = w.head_size ** -0.5
    if run.mode == "int4":
        ref = O.paged_attention(q, kc, vc, ks, vs, bt, lay.seq_lens, lay.query_start_loc, scale, w.sign_seed,
                                seqs=[s], window=run.window)[q0:q1]
    else:
        ref = O.pth_paged_attention(q, kc, vc, ks, vs, bt, lay.seq_lens, lay.query_start_loc, scale, run.mode,
                                    seqs=[s], window=run.window)[q0:q1]
    L = int(w.seq_lens[s])
    dense = O.attention_dense(q[q0:q1], k_raw, v_raw, np.array([0, q1 - q0]), [L], scale, np.array([0, L]),
                              window=run.window)
    return s, ref, dense


def test_full_size_attention(full: FullRun):
    """G2 on every query row; G4 reported on every row and asserted where the
    oracle's own quantized result meets it (see the module docstring)."""
    w, lay = full.w, full.lay
    q = W.bf16_as_f32_numpy(full.query)
    got = host(full.out.float())
    assert np.isfinite(got).all()
    ref = np.zeros(got.shape)
    dense = np.zeros(got.shape)
    pool, limit = _pool()
    futs, results = [], []
    with pool, limit:
        for s in range(w.num_seqs):
            if lay.query_start_loc[s + 1] == lay.query_start_loc[s]:
                continue
            k0, L = int(lay.kv_start[s]), int(w.seq_lens[s])
            k_raw = W.bf16_as_f32_numpy(full.key[k0:k0 + L])
            v_raw = W.bf16_as_f32_numpy(full.value[k0:k0 + L])
            futs.append(pool.submit(_attn_job, full, s, q, _seq_pages(full, s), k_raw, v_raw))
            _drain(futs, results, 2 * worker_count())
        _drain(futs, results, 0)
    for s, r, d in results:
        q0, q1 = int(lay.query_start_loc[s]), int(lay.query_start_loc[s + 1])
        ref[q0:q1], dense[q0:q1] = r, d

    err2 = np.abs(got - ref)
    bad2 = int(np.count_nonzero(err2 > G2_TOL + G2_TOL * np.abs(ref)))
    tol4 = G4_TOL + G4_TOL * np.abs(dense)
    slack_o = (np.abs(ref - dense) / tol4).max(axis=-1)                  # per (query row, q head)
    slack_g = (np.abs(got - dense) / tol4).max(axis=-1)
    sel = slack_o <= G4_ASSERT_SLACK
    bad4 = int(np.count_nonzero(slack_g[sel] > 1.0))

    def corr(a, b):
        return float(np.corrcoef(a.ravel(), b.ravel())[0, 1])

    say(f"    G2 over {got.shape[0]} query rows x {w.num_q_heads} heads: max abs err {err2.max():.3e}, "
        f"violations {bad2}")
    say(f"    G4 vs unquantized fp64: GPU max abs err {np.abs(got - dense).max():.3e} corr {corr(got, dense):.5f}; "
        f"oracle max abs err {np.abs(ref - dense).max():.3e} corr {corr(ref, dense):.5f}; "
        f"oracle misses 5e-2 on {int(np.count_nonzero(slack_o > 1))} of {slack_o.size} rows; asserted on "
        f"{int(sel.sum())} rows, GPU violations there {bad4}")
    assert bad2 == 0
    assert bad4 == 0
