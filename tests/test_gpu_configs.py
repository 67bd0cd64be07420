"""Parity at the full workload sizes the benchmark runs (Phi-3 hs 96,
Llama-3.2-1B GQA, Qwen2.5-1.5B mixed prefill+decode, Llama-3-8B long context
hs 128 and hs 192), in the same launch configuration: every KV token written
in one kv4_rht_write call, one kv4_paged_attention call over the batch.

Sampled checks the oracle can finish in seconds: codes and scales of 4096
random tokens bit-exact (G1); attention outputs of a sample of sequences
(the longest, the shortest and random ones, every prefill sequence) within
atol = rtol = 1e-2 of the fp64 oracle reading the GPU-written cache (G2)."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, O, W, allclose_report, host, run_gpu, say

pytestmark = pytest.mark.gpu

CONFIGS = ["phi3", "llama1b", "qwen_mixed", "llama8b_long", "llama8b_hs192"]


def _sample_g1(r, n=4096):
    w = r.w
    T = r.slots.shape[0]
    rows = np.sort(np.random.default_rng(0).choice(T, size=min(n, T), replace=False))
    idx = torch.from_numpy(rows).to(r.t.key.device)
    key = W.bf16_as_f32_numpy(r.t.key.index_select(0, idx))
    value = W.bf16_as_f32_numpy(r.t.value.index_select(0, idx))
    sl = r.slots[rows]
    bs = w.block_size
    d = O.rht_signs(w.sign_seed, w.head_size)
    slt = torch.from_numpy(sl).to(DEV)
    for x, c, s in ((key, r.kc, r.ks), (value, r.vc, r.vs)):
        codes, scale = O.quantize_int4(O.rotate_spec(x, d))
        got_c = host(c.view(-1, w.num_kv_heads, w.head_size // 2).index_select(0, slt))
        got_s = host(s.view(-1, w.num_kv_heads).index_select(0, slt))
        np.testing.assert_array_equal(got_c, O.pack_int4(codes))
        np.testing.assert_array_equal(got_s.view(np.uint32), scale.view(np.uint32))


def _sample_seqs(w, k=6):
    L = np.asarray(w.seq_lens)
    q = np.asarray(w.query_lens)
    pick = {int(np.argmax(L)), int(np.argmin(L))}
    pick |= set(int(i) for i in np.nonzero(q > 1)[0])
    rng = np.random.default_rng(1)
    pick |= set(int(i) for i in rng.choice(len(L), size=min(k, len(L)), replace=False))
    return sorted(pick)


def _gather_seq_cache(r, seqs):
    """Copy only the pages of the sampled sequences to the host (renumbered)."""
    w = r.w
    pages = sorted({int(p) for s in seqs for p in r.lay.block_table[s, :(-(-w.seq_lens[s] // w.block_size))]})
    remap = {p: i for i, p in enumerate(pages)}
    pt = torch.tensor(pages, dtype=torch.int64, device=DEV)
    kc, vc = host(r.kc.index_select(0, pt)), host(r.vc.index_select(0, pt))
    ks, vs = host(r.ks.index_select(0, pt)), host(r.vs.index_select(0, pt))
    bt = np.zeros_like(r.lay.block_table)
    for s in seqs:
        n = -(-w.seq_lens[s] // w.block_size)
        bt[s, :n] = [remap[int(p)] for p in r.lay.block_table[s, :n]]
    return kc, vc, ks, vs, bt


@pytest.mark.parametrize("name", CONFIGS)
def test_full_size_config(name):
    w = W.ALL[name]()
    r = run_gpu(w, gen_device=DEV)
    say(f"    written {w.total_kv_tokens} tokens; checking G1 on a sample")
    _sample_g1(r)
    seqs = _sample_seqs(w)
    kc, vc, ks, vs, bt = _gather_seq_cache(r, seqs)
    q = W.bf16_as_f32_numpy(r.t.query)
    ref = O.paged_attention(q, kc, vc, ks, vs, bt, r.lay.seq_lens, r.lay.query_start_loc,
                            w.head_size ** -0.5, w.sign_seed, seqs=seqs)
    got = host(r.out.float())
    rows = np.concatenate([np.arange(r.lay.query_start_loc[s], r.lay.query_start_loc[s + 1]) for s in seqs])
    nbad, mx = allclose_report(got[rows], ref[rows], atol=1e-2, rtol=1e-2)
    say(f"    G2 on {len(seqs)} sequences ({len(rows)} query rows): max abs err {mx:.3e}, violations {nbad}")
    assert nbad == 0
    assert np.isfinite(got).all()
