"""Benchmark of the INT4 per-token-head RHT KV-cache hot path on one MI355X.

One step = one serving step of the hot path over a resident batch: the step's
new K/V tokens go through kv4_rht_write (rotate, round through bf16,
quantize, pack, scatter) and then kv4_paged_attention runs over the whole
batch (query rotation, paged int4 KV stream with on-the-fly dequant, online
softmax with softmax_scale / b, split merge, inverse rotation of the output).
Inputs are synthetic and seeded (workloads/), already in HBM when the timed
region starts; the context of every sequence is written before timing with
the same write kernel (that bulk write is timed separately and reported as
write tokens/s).

Prints ONE JSON line. `value` is decode-attention KV GB/s: algorithmic bytes
the step's attention must read (int4 codes + fp32 scales of every visible
(KV token, kv head), page-table entries, query and output) divided by the
step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
CSRC = os.path.join(ROOT, "paged_decode_attention_reshape_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def code_bytes(w, mode: str) -> int:
    """Code bytes of one (token, kv head) row of one cache: int4 packs two
    codes per byte; int8 / fp8 take one byte per element."""
    return w.head_size // 2 if mode == "int4" else w.head_size


def visible_keys(w, window: int = 0):
    """Per sequence, the keys some query of it can see: all L, or with a
    sliding window the last window + query_len - 1 of them."""
    if window <= 0:
        return list(w.seq_lens)
    return [min(L, window + q - 1) if q > 0 else 0 for L, q in zip(w.seq_lens, w.query_lens)]


def attention_bytes(w, mode: str = "int4", window: int = 0) -> int:
    """Algorithmic bytes one attention pass must move: for every sequence,
    every visible (KV token, kv head): the K and V code rows + 2 fp32 scales;
    plus block-table entries, bf16 query in and bf16 output out."""
    vis = visible_keys(w, window)
    kv = int(sum(vis) * w.num_kv_heads * (2 * code_bytes(w, mode) + 8))
    bt = sum(-(-n // w.block_size) for n in vis) * 4
    qo = w.num_q_tokens * w.num_q_heads * w.head_size * 2 * 2
    return int(kv + bt + qo)


def kv_bytes(w, mode: str = "int4") -> int:
    return int(sum(w.seq_lens) * w.num_kv_heads * (2 * code_bytes(w, mode) + 8))


def write_bytes_per_token(w, mode: str = "int4") -> int:
    """Read bf16 K and V, write the codes and two fp32 scales per kv head,
    read one int64 slot."""
    return w.num_kv_heads * (4 * w.head_size + 2 * code_bytes(w, mode) + 8) + 8


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama8b_long")
    ap.add_argument("--kv-mode", default="int4", choices=["int4", "int8", "fp8"],
                    help="cache format: int4 RHT (the method) or the per-token-head int8 / fp8 controls")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window (keys per query; 0 = full causal attention)")
    ap.add_argument("--layout", default="packed", choices=["packed", "inline"],
                    help="cache layout: separate packed code and scale tensors, or one buffer with each "
                         "row's scale inline and rows padded to 16 bytes")
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of back-to-back steps before the warmup steps, so that the GPU's clocks have "
                         "left their idle state (a serving GPU runs continuously); never timed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) -- the reference "
                         "kernel of known size for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path here "
              "(the write path and attention would shard by kv head or sequence with no exchange). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_decode_attention_reshape_amd as kv4
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        # a read-only pass over the same bytes (float32 sum: reads n bytes, writes one value)
        f = src.view(torch.float32)
        for _ in range(5):
            f.sum()
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "repeats": 5}))
        return
    w = W.ALL[args.config]()
    lay = W.make_layout(w)
    print(f"# config {w.name}: seqs={w.num_seqs} nq={w.num_q_heads} nkv={w.num_kv_heads} hs={w.head_size} "
          f"kv_tokens={w.total_kv_tokens} q_tokens={w.num_q_tokens}", file=sys.stderr, flush=True)
    t = W.make_tensors(w, lay, device=dev)
    slots_all = W.all_slots(lay, w)
    new_rows = W.new_token_rows(lay, w)
    ctx_mask = np.ones(slots_all.shape[0], dtype=bool)
    ctx_mask[new_rows] = False
    ctx_rows = np.nonzero(ctx_mask)[0]

    nb, bs, nkv, hs = lay.num_blocks, w.block_size, w.num_kv_heads, w.head_size
    mode = args.kv_mode
    inline = args.layout == "inline" or args.window > 0
    if args.layout == "inline":
        lcache = kv4.LayoutCache.inline(mode, nb, bs, nkv, hs, device=dev)
        kc = vc = ks = vs = None
    else:
        kc = torch.zeros((nb, bs, nkv, code_bytes(w, mode)), dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb, bs, nkv), dtype=torch.float32, device=dev)
        vs = torch.zeros_like(ks)
        if inline:    # packed caches through the layout entry points (sliding window)
            lcache = kv4.packed_layout_cache(mode, kc, vc, ks, vs)
    stream = torch.cuda.Stream()

    def write(k, v, slots):
        if inline:
            kv4.kv4_write_layout(k, v, lcache, slots, sign_seed=w.sign_seed, stream=stream)
        elif mode == "int4":
            kv4.kv4_rht_write(k, v, kc, vc, ks, vs, slots, sign_seed=w.sign_seed, stream=stream)
        else:
            kv4.kv4_pth_write(mode, k, v, kc, vc, ks, vs, slots, stream=stream)

    # ---- bulk write of every context token (here untimed; timed again after
    # the pre-warm below)
    ctx_idx = torch.from_numpy(ctx_rows).to(dev)
    k_ctx = t.key.index_select(0, ctx_idx)
    v_ctx = t.value.index_select(0, ctx_idx)
    s_ctx = torch.from_numpy(slots_all[ctx_rows]).to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        write(k_ctx, v_ctx, s_ctx)
    torch.cuda.synchronize()
    n_ctx = int(ctx_rows.shape[0])

    # ---- step inputs
    new_idx = torch.from_numpy(new_rows).to(dev)
    k_new = t.key.index_select(0, new_idx).contiguous()
    v_new = t.value.index_select(0, new_idx).contiguous()
    s_new = torch.from_numpy(slots_all[new_rows]).to(dev)
    q = t.query
    bt = torch.from_numpy(lay.block_table).to(dev)
    slens = torch.from_numpy(lay.seq_lens).to(dev)
    qsl = torch.from_numpy(lay.query_start_loc).to(dev)
    out = torch.empty((w.num_q_tokens, w.num_q_heads, hs), dtype=torch.bfloat16, device=dev)
    if inline:
        need = kv4.kv4_attention_layout_workspace_size(lcache, w.num_q_tokens, w.num_seqs, w.num_q_heads,
                                                       w.max_query_len, w.max_seq_len)
    elif mode == "int4":
        need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads, nkv, hs,
                                                      w.max_query_len, w.max_seq_len)
    else:
        need = kv4.kv4_pth_attention_workspace_size(mode, w.num_q_tokens, w.num_seqs, w.num_q_heads, nkv, hs,
                                                    w.max_query_len, w.max_seq_len)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def step(e_a=None, e_b=None):
        write(k_new, v_new, s_new)
        if e_a is not None:
            e_a.record(stream)
        if inline:
            kv4.kv4_attention_layout(q, lcache, bt, slens, qsl, w.max_query_len, w.max_seq_len,
                                     sign_seed=w.sign_seed, out=out, workspace=ws, stream=stream,
                                     sliding_window=args.window)
        elif mode == "int4":
            kv4.kv4_paged_attention(q, kc, vc, ks, vs, bt, slens, qsl, max_query_len=w.max_query_len,
                                    max_seq_len=w.max_seq_len, sign_seed=w.sign_seed, out=out, workspace=ws,
                                    stream=stream)
        else:
            kv4.kv4_pth_attention(mode, q, kc, vc, ks, vs, bt, slens, qsl, max_query_len=w.max_query_len,
                                  max_seq_len=w.max_seq_len, out=out, workspace=ws, stream=stream)
        if e_b is not None:
            e_b.record(stream)

    # Clock ramp: a few milliseconds of work leave the GPU below its steady
    # clocks (measured at the Llama-3-8B shape: 5 warmup steps 4.8-5.0 TB/s,
    # 200 warmup steps 5.4 TB/s for the same timed steps), so steps run back to
    # back for --prewarm-s seconds first. Untimed, like the warmup steps.
    prewarm_steps = 0
    t_pre = time.perf_counter() + max(args.prewarm_s, 0.0)
    with torch.cuda.stream(stream):
        while time.perf_counter() < t_pre:
            for _ in range(8):
                step()
            prewarm_steps += 8
            stream.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(ev_a[i], ev_b[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [ev_a[i].elapsed_time(ev_b[i]) for i in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps
    attn_avg_ms = float(np.mean(attn_ms))

    # The bulk write again, timed at steady clocks (same values into the same
    # slots), after the timed steps: three full context writes right before
    # them left the attention steps 4-9 % slower for the rest of the process
    # (measured at the Llama-3-8B shape, whatever the pre-warm in between).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    wr_ms = []
    with torch.cuda.stream(stream):
        for rep in range(3):
            ev[0].record(stream)
            write(k_ctx, v_ctx, s_ctx)
            ev[1].record(stream)
            stream.synchronize()
            wr_ms.append(ev[0].elapsed_time(ev[1]))
    del k_ctx, v_ctx
    write_ms = float(np.median(wr_ms))
    write_tps = n_ctx / (write_ms * 1e-3) if n_ctx else 0.0
    write_gbs = n_ctx * write_bytes_per_token(w, mode) / (write_ms * 1e-3) / 1e9 if n_ctx else 0.0
    a_bytes = attention_bytes(w, mode, args.window)
    value = a_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = a_bytes / (attn_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        try:
            pc = json.load(open(PROFILE_COUNTERS))
            key = (w.name + ("" if mode == "int4" else f"_{mode}") + ("_inline" if args.layout == "inline" else "")
                   + (f"_w{args.window}" if args.window > 0 else ""))
            ent = pc.get("workloads", {}).get(key)
            if ent and pc.get("kernel_source_hash") == kernel_source_hash():
                traffic = ent.get("traffic_bytes_per_launch")
        except Exception:
            traffic = None

    line = {
        "metric": "INT4 paged decode attn: KV GB/s & % HBM peak; cache-write tokens/s"
                  + ("" if mode == "int4" else f" ({mode} per-token-head control cache)")
                  + (" (inline-scale padded-slot layout)" if args.layout == "inline" else "")
                  + (f" (sliding window {args.window})" if args.window > 0 else ""),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": prewarm_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{mode} codes / fp32 accumulate (bf16 in/out)",
        "data": "synthetic seeded N(0,1) bf16, 1% outlier channels x20",
        "config": {"workload": w.name, "kv_cache": mode, "cache_layout": args.layout,
                   "sliding_window": args.window, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": nkv, "head_size": hs, "block_size": bs,
                   "total_kv_tokens": w.total_kv_tokens, "max_seq_len": w.max_seq_len,
                   "q_tokens_per_step": w.num_q_tokens, "new_kv_tokens_per_step": int(new_rows.shape[0]),
                   "parallelism": "single GPU"},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "attn_ms": round(attn_avg_ms, 4),
        "attn_query_tokens_per_s": round(w.num_q_tokens / (attn_avg_ms * 1e-3), 1),
        "kv_bytes_per_step": int(sum(visible_keys(w, args.window)) * w.num_kv_heads * (2 * code_bytes(w, mode) + 8)),
        "write_tokens_per_s": round(write_tps, 1),
        "write_GBps": round(write_gbs, 2),
        "write_bulk_tokens": n_ctx,
        "roofline": {"bound": "hbm", "kernel": ("kv4_paged_attention" if mode == "int4" else "kv4_pth_attention")
                     + " (attention + merge)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": a_bytes},
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, lay, t, kc, vc, ks, vs, args.cpu_seconds, mode,
                                            lcache if args.layout == "inline" else None, args.window)
    print(json.dumps(line), flush=True)


def cpu_baseline(w, lay, t, kc, vc, ks, vs, budget_s: float, mode: str = "int4", lcache=None, window: int = 0):
    """The CPU oracle (fp64 numpy) on a bounded sample of the same workload:
    whole sequences of this batch, read from the GPU-written cache, until
    about `budget_s` seconds of CPU work; reported as KV GB/s like `value`."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import kv4_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    order = np.random.default_rng(0).permutation(w.num_seqs)
    q = W.bf16_as_f32_numpy(t.query)
    done_bytes, done_seqs, spent = 0, 0, 0.0
    dev = (lcache.buffer if lcache is not None else kc).device
    for s in order:
        n = -(-w.seq_lens[s] // w.block_size)
        pages = torch.from_numpy(lay.block_table[s, :n].astype(np.int64)).to(dev)
        if lcache is not None:     # the sequence's pages of the inline buffer, unpacked (not timed)
            kcs, vcs, kss, vss = O.inline_unpack(lcache.buffer.index_select(0, pages).cpu().numpy(), mode,
                                                 w.num_kv_heads, w.head_size, w.block_size)
        else:
            kcs, vcs = kc.index_select(0, pages).cpu().numpy(), vc.index_select(0, pages).cpu().numpy()
            kss, vss = ks.index_select(0, pages).cpu().numpy(), vs.index_select(0, pages).cpu().numpy()
        bt = np.zeros_like(lay.block_table)
        bt[s, :n] = np.arange(n)
        t0 = time.perf_counter()
        if mode == "int4":
            O.paged_attention(q, kcs, vcs, kss, vss, bt, lay.seq_lens, lay.query_start_loc,
                              w.head_size ** -0.5, w.sign_seed, seqs=[int(s)], window=window)
        else:
            O.pth_paged_attention(q, kcs, vcs, kss, vss, bt, lay.seq_lens, lay.query_start_loc,
                                  w.head_size ** -0.5, mode, seqs=[int(s)], window=window)
        spent += time.perf_counter() - t0
        done_bytes += int(visible_keys(w, window)[s]) * w.num_kv_heads * (2 * code_bytes(w, mode) + 8)
        done_seqs += 1
        if spent >= budget_s:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done_seqs} of {w.num_seqs} sequences of {w.name} (fp64 numpy oracle reading the "
                      f"GPU-written cache), {spent:.1f} s of CPU time"}


if __name__ == "__main__":
    main()
