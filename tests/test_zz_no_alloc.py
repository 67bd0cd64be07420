"""kv4_paged_attention_noalloc (static per-GPU scratch, no allocation)
against kv4_paged_attention (caller workspace) on the same inputs: two calls
in a row, the second with a smaller batch, each bit-identical to the
workspace entry point (same plan, same kernels) and within G2 of the oracle;
and a batch that needs more than the static scratch is refused before any
launch."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, W, allclose_report, host, kv4, oracle_attention_on_gpu_cache, run_gpu, say

pytestmark = pytest.mark.gpu


def _both(w):
    r = run_gpu(w)                                    # kv4_paged_attention with the binding's workspace
    lay = r.lay
    bt, slens, qsl = (torch.from_numpy(x).to(DEV) for x in (lay.block_table, lay.seq_lens, lay.query_start_loc))
    out = torch.full((w.num_q_tokens, w.num_q_heads, w.head_size), 5.0, dtype=torch.bfloat16, device=DEV)
    kv4.kv4_paged_attention_noalloc(r.t.query.to(DEV), r.kc, r.vc, r.ks, r.vs, bt, slens, qsl,
                                    max_query_len=w.max_query_len, max_seq_len=w.max_seq_len, out=out,
                                    sign_seed=w.sign_seed)
    torch.cuda.synchronize()
    return r, out


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [
        # stream-K decode, GQA 4, several thousand keys: partials in the scratch
        W.custom("noalloc_big", 32, 8, 128, [1] * 24, [int(x) for x in np.linspace(40, 9000, 24)],
                 outlier_frac=0.01),
        # then a smaller batch of another shape (head size 96, split-KV multi-token tiles)
        W.custom("noalloc_small", 8, 2, 96, [3, 1, 5], [700, 33, 260], seed=3),
    ]
    for w in cases:
        need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads,
                                                      w.num_kv_heads, w.head_size, w.max_query_len,
                                                      w.max_seq_len)
        assert 0 < need <= kv4.KV4_NOALLOC_SCRATCH_BYTES
        r, out = _both(w)
        got = host(out.float())
        assert np.array_equal(got, host(r.out.float())), "noalloc differs from the workspace entry point"
        ref = oracle_attention_on_gpu_cache(r)
        nbad, mx = allclose_report(got, ref, atol=1e-2, rtol=1e-2)
        say(f"    {w.name}: workspace {need} B; bit-identical; G2 max abs err {mx:.3e}")
        assert nbad == 0


def test_noalloc_with_the_prefill_kernel(monkeypatch):
    """A mixed chunked-prefill batch on the prefill kernel (its decode rows'
    partials and both prefixes in the scratch; no side stream), then a smaller
    decode batch: bit-identical to the workspace entry point, within G2."""
    monkeypatch.setenv("KV4_PREFILL", "1")
    cases = [
        W.custom("noalloc_pf", 12, 2, 128, [150, 1, 1, 40, 1], [2000, 3000, 70, 400, 900], seed=5),
        W.custom("noalloc_pf_small", 16, 4, 128, [1, 1], [300, 1000], seed=6),
    ]
    for w in cases:
        need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads,
                                                      w.num_kv_heads, w.head_size, w.max_query_len,
                                                      w.max_seq_len)
        assert 0 < need <= kv4.KV4_NOALLOC_SCRATCH_BYTES
        r, out = _both(w)
        got = host(out.float())
        assert np.array_equal(got, host(r.out.float())), "noalloc differs from the workspace entry point"
        ref = oracle_attention_on_gpu_cache(r)
        nbad, mx = allclose_report(got, ref, atol=1e-2, rtol=1e-2)
        say(f"    {w.name}: workspace {need} B; bit-identical; G2 max abs err {mx:.3e}")
        assert nbad == 0


def test_noalloc_fits_the_tile_launch_to_the_scratch():
    """A Qwen2.5-1.5B-shaped mixed batch (4 chunks of 512, 60 four-query
    sequences, 4 decodes) whose workspace, as the caller's workspace entry
    point plans it, exceeds the static scratch: the launch of the
    four-query sequences beside the prefill kernel takes longer key pieces
    until the call fits. Its rows then merge fewer partials, so the output
    agrees with the workspace entry point to the fp32 accumulation order
    (within G2) rather than bit for bit; every row is within G2 of the
    oracle."""
    rng = np.random.default_rng(11)
    ql = [512] * 4 + [4] * 60 + [1] * 4
    sl = [2560] * 4 + [int(x) for x in np.exp(rng.uniform(np.log(256), np.log(8192), 64))]
    order = rng.permutation(len(ql))
    w = W.custom("noalloc_fit", 12, 2, 128, [ql[i] for i in order], [sl[i] for i in order], seed=7)
    need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                  w.head_size, w.max_query_len, w.max_seq_len)
    assert need > kv4.KV4_NOALLOC_SCRATCH_BYTES
    r, out = _both(w)
    got = host(out.float())
    nbad, mx = allclose_report(got, host(r.out.float()), atol=1e-2, rtol=1e-2)
    assert nbad == 0, f"noalloc against the workspace entry point: {nbad} elements (max {mx})"
    ref = oracle_attention_on_gpu_cache(r)
    nbad, mx = allclose_report(got, ref, atol=1e-2, rtol=1e-2)
    say(f"    {w.name}: planned workspace {need} B > scratch; G2 max abs err {mx:.3e}")
    assert nbad == 0


def test_noalloc_refuses_batches_beyond_the_scratch(monkeypatch):
    # the mixed chunked-prefill batch on the single-kernel plan (its split
    # partials over all 2108 query tokens: ~118 MB)
    monkeypatch.setenv("KV4_PREFILL", "0")
    w = W.ALL["qwen_mixed"]()
    need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                  w.head_size, w.max_query_len, w.max_seq_len)
    assert need > kv4.KV4_NOALLOC_SCRATCH_BYTES
    r = run_gpu(w, attention=False)
    lay = r.lay
    bt, slens, qsl = (torch.from_numpy(x).to(DEV) for x in (lay.block_table, lay.seq_lens, lay.query_start_loc))
    out = torch.full((w.num_q_tokens, w.num_q_heads, w.head_size), 5.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kv4.Kv4Error) as ei:
        kv4.kv4_paged_attention_noalloc(r.t.query.to(DEV), r.kc, r.vc, r.ks, r.vs, bt, slens, qsl,
                                        max_query_len=w.max_query_len, max_seq_len=w.max_seq_len, out=out,
                                        sign_seed=w.sign_seed)
    assert ei.value.code == kv4.KV4_EWORKSPACE and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert host(out.float()).min() == 5.0 and host(out.float()).max() == 5.0   # nothing was launched
