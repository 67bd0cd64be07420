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
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak (no sparsity)
MALL_ROTATE_BELOW = 512 << 20  # working sets below this are rotated through copies (256 MB Infinity Cache)
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


def attention_flops(w, window: int = 0) -> int:
    """Algorithmic flops of one attention pass: 4 * head_size per (query
    head, visible key) -- q.k and p.v, a multiply and an add each. Query i of a
    sequence with query_len q and seq_len L sees the keys at positions up to
    L - q + i (and with a window only the last `window` of them)."""
    pairs = 0
    for L, q in zip(w.seq_lens, w.query_lens):
        for i in range(q):
            vis = max(0, L - q + i + 1)
            pairs += min(vis, window) if window > 0 else vis
    return int(4 * w.head_size * w.num_q_heads * pairs)


def percentile(xs, p: float) -> float:
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), p))


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
    ap.add_argument("--rotate", type=int, default=0, metavar="N",
                    help="independent copies of the cache the steps cycle through, so that a working set "
                         "smaller than the 256 MB Infinity Cache is not served from it by the previous step "
                         "(as in a model, where the other layers' caches pass in between); 0 = 4 copies when "
                         "the step's KV working set is below 512 MB, else 1")
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of back-to-back steps before the warmup steps, so that the GPU's clocks have "
                         "left their idle state (a serving GPU runs continuously); never timed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the measured HBM read ceiling (kv4_stream_read over 2 GiB)")
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
    use_layout = args.layout == "inline" or args.window > 0
    kv_set = int(sum(visible_keys(w, args.window)) * nkv * (2 * code_bytes(w, mode) + 8))
    n_copies = args.rotate if args.rotate > 0 else (4 if kv_set < MALL_ROTATE_BELOW else 1)

    def new_cache():
        """One cache set: (packed tensors or None, layout cache or None)."""
        if args.layout == "inline":
            return None, kv4.LayoutCache.inline(mode, nb, bs, nkv, hs, device=dev)
        kc = torch.zeros((nb, bs, nkv, code_bytes(w, mode)), dtype=torch.uint8, device=dev)
        packed = (kc, torch.zeros_like(kc), torch.zeros((nb, bs, nkv), dtype=torch.float32, device=dev),
                  torch.zeros((nb, bs, nkv), dtype=torch.float32, device=dev))
        # packed caches through the layout entry points (sliding window)
        return packed, (kv4.packed_layout_cache(mode, *packed) if use_layout else None)

    caches = [new_cache() for _ in range(n_copies)]
    stream = torch.cuda.Stream()

    def write(c, k, v, slots):
        packed, lcache = c
        if lcache is not None:
            kv4.kv4_write_layout(k, v, lcache, slots, sign_seed=w.sign_seed, stream=stream)
        elif mode == "int4":
            kv4.kv4_rht_write(k, v, *packed, slots, sign_seed=w.sign_seed, stream=stream)
        else:
            kv4.kv4_pth_write(mode, k, v, *packed, slots, stream=stream)

    # ---- bulk write of every context token into every copy (here untimed;
    # timed again after the timed steps)
    ctx_idx = torch.from_numpy(ctx_rows).to(dev)
    k_ctx = t.key.index_select(0, ctx_idx)
    v_ctx = t.value.index_select(0, ctx_idx)
    s_ctx = torch.from_numpy(slots_all[ctx_rows]).to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for c in caches:
            write(c, k_ctx, v_ctx, s_ctx)
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
    if use_layout:
        need = kv4.kv4_attention_layout_workspace_size(caches[0][1], w.num_q_tokens, w.num_seqs, w.num_q_heads,
                                                       w.max_query_len, w.max_seq_len)
    elif mode == "int4":
        need = kv4.kv4_paged_attention_workspace_size(w.num_q_tokens, w.num_seqs, w.num_q_heads, nkv, hs,
                                                      w.max_query_len, w.max_seq_len)
    else:
        need = kv4.kv4_pth_attention_workspace_size(mode, w.num_q_tokens, w.num_seqs, w.num_q_heads, nkv, hs,
                                                    w.max_query_len, w.max_seq_len)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    step_no = [0]

    def step(e_a=None, e_b=None):
        packed, lcache = caches[step_no[0] % n_copies]
        step_no[0] += 1
        write((packed, lcache), k_new, v_new, s_new)
        if e_a is not None:
            e_a.record(stream)
        if lcache is not None:
            kv4.kv4_attention_layout(q, lcache, bt, slens, qsl, w.max_query_len, w.max_seq_len,
                                     sign_seed=w.sign_seed, out=out, workspace=ws, stream=stream,
                                     sliding_window=args.window)
        elif mode == "int4":
            kv4.kv4_paged_attention(q, *packed, bt, slens, qsl, max_query_len=w.max_query_len,
                                    max_seq_len=w.max_seq_len, sign_seed=w.sign_seed, out=out, workspace=ws,
                                    stream=stream)
        else:
            kv4.kv4_pth_attention(mode, q, *packed, bt, slens, qsl, max_query_len=w.max_query_len,
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
            write(caches[rep % n_copies], k_ctx, v_ctx, s_ctx)
            ev[1].record(stream)
            stream.synchronize()
            wr_ms.append(ev[0].elapsed_time(ev[1]))
    del k_ctx, v_ctx
    write_ms = float(np.median(wr_ms))
    write_tps = n_ctx / (write_ms * 1e-3) if n_ctx else 0.0
    write_gbs = n_ctx * write_bytes_per_token(w, mode) / (write_ms * 1e-3) / 1e9 if n_ctx else 0.0
    a_bytes = attention_bytes(w, mode, args.window)
    a_flops = attention_flops(w, args.window)
    value = a_bytes / (ms_per_step * 1e-3) / 1e9

    # Roofline of the attention call: the larger of its time at the HBM peak
    # (algorithmic bytes) and at the matrix-core peak (algorithmic flops)
    # decides the bound; achieved is taken over the mean HIP-event time of
    # the call on its stream (what a kernel trace averages).
    t_hbm = a_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = a_flops / (MFMA_PEAK_TFLOPS * 1e12)
    gbs = a_bytes / (attn_avg_ms * 1e-3) / 1e9
    tflops = a_flops / (attn_avg_ms * 1e-3) / 1e12
    bound = "mfma" if t_mfma > t_hbm else "hbm"

    read_ceiling = None
    if not args.no_read_ceiling:
        read_ceiling = measured_read_ceiling(torch, kv4, dev, stream)

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

    roof = {"bound": bound,
            "kernel": ("kv4_paged_attention" if mode == "int4" and not use_layout else
                       "kv4_attention_layout" if use_layout else "kv4_pth_attention") + " (attention + merge)",
            "achieved": round(tflops if bound == "mfma" else gbs, 2),
            "peak": MFMA_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round((tflops / MFMA_PEAK_TFLOPS) if bound == "mfma" else (gbs / HBM_PEAK_GBS), 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": a_bytes,
            "algorithmic_flops_per_launch": a_flops,
            "time_at_hbm_peak_us": round(t_hbm * 1e6, 2),
            "time_at_mfma_peak_us": round(t_mfma * 1e6, 2),
            "hbm_GBps": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_TFLOPs": round(tflops, 2), "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4)}
    if read_ceiling:
        roof["measured_read_GBps"] = read_ceiling["GBps"]
        roof["hbm_frac_of_measured"] = round(gbs / read_ceiling["GBps"], 4)

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
        "data": "synthetic seeded N(0,1) bf16" + (", 1% outlier channels x20" if w.outlier_frac > 0 else ""),
        "config": {"workload": w.name, "kv_cache": mode, "cache_layout": args.layout,
                   "sliding_window": args.window, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": nkv, "head_size": hs, "block_size": bs,
                   "total_kv_tokens": w.total_kv_tokens, "max_seq_len": w.max_seq_len,
                   "q_tokens_per_step": w.num_q_tokens, "new_kv_tokens_per_step": int(new_rows.shape[0]),
                   "cache_copies_rotated": n_copies, "parallelism": "single GPU"},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "attn_ms": round(attn_avg_ms, 4),
        "attn_ms_median": round(percentile(attn_ms, 50), 4),
        "attn_ms_p10": round(percentile(attn_ms, 10), 4),
        "attn_ms_p90": round(percentile(attn_ms, 90), 4),
        "attn_GBps_median": round(a_bytes / (percentile(attn_ms, 50) * 1e-3) / 1e9, 2),
        "attn_query_tokens_per_s": round(w.num_q_tokens / (attn_avg_ms * 1e-3), 1),
        "kv_bytes_per_step": kv_set,
        "write_tokens_per_s": round(write_tps, 1),
        "write_GBps": round(write_gbs, 2),
        "write_hbm_frac": round(write_gbs / HBM_PEAK_GBS, 4),
        "write_bulk_tokens": n_ctx,
        "roofline": roof,
    }
    if read_ceiling:
        line["read_ceiling"] = read_ceiling

    if not args.no_cpu_baseline:
        packed0, lcache0 = caches[0]
        kc, vc, ks, vs = packed0 if packed0 is not None else (None,) * 4
        line["cpu_baseline"] = cpu_baseline(w, lay, t, kc, vc, ks, vs, args.cpu_seconds, mode,
                                            lcache0 if args.layout == "inline" else None, args.window,
                                            ctx_rows, slots_all)
    print(json.dumps(line), flush=True)


def measured_read_ceiling(torch, kv4, dev, stream, nbytes: int = 2 << 30):
    """Achievable HBM read rate on this GPU: kv4_stream_read over a 2 GiB
    buffer (8x the Infinity Cache) at three grid sizes, 3 warm + 10 timed
    passes each; the best median, with its spread."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = None
    for grid in (1024, 2048, 4096):
        ms = []
        with torch.cuda.stream(stream):
            for rep in range(13):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                kv4.kv4_stream_read(buf, sink, grid=grid, stream=stream)
                e1.record(stream)
                stream.synchronize()
                if rep >= 3:
                    ms.append(e0.elapsed_time(e1))
        med = percentile(ms, 50)
        ent = {"GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "grid": grid,
               "GBps_p10_p90": [round(nbytes / (percentile(ms, 90) * 1e-3) / 1e9, 1),
                                round(nbytes / (percentile(ms, 10) * 1e-3) / 1e9, 1)]}
        if best is None or ent["GBps"] > best["GBps"]:
            best = ent
    del buf
    best["kernel"] = "kv4_stream_read (16-byte non-temporal loads, 2 GiB, median of 10)"
    return best


def cpu_baseline(w, lay, t, kc, vc, ks, vs, budget_s: float, mode: str = "int4", lcache=None, window: int = 0,
                 ctx_rows=None, slots_all=None):
    """The CPU oracle (numpy) on a bounded sample of the same workload:
    attention over whole sequences of this batch, read from the GPU-written
    cache, until about `budget_s` seconds of CPU work (reported as KV GB/s
    like `value`, and as query tokens/s); and the write path (spec tier:
    rotation, bf16 rounding, quantization, packing) on the first context
    tokens for about a fifth of that (tokens/s)."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import kv4_oracle as O

    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = sorted({f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                       for i in info if i.get("user_api") == "blas"})
    except Exception:  # pragma: no cover
        threads, blas = 1, []
    order = np.random.default_rng(0).permutation(w.num_seqs)
    q = W.bf16_as_f32_numpy(t.query)
    done_bytes, done_seqs, done_q, spent = 0, 0, 0, 0.0
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
        done_q += int(w.query_lens[s])
        if spent >= budget_s:
            break

    # write path: chunks of 4096 context tokens (K and V) until the budget
    wr_tok, wr_spent = 0, 0.0
    if ctx_rows is not None and len(ctx_rows):
        nb = lay.num_blocks
        for r0 in range(0, len(ctx_rows), 4096):
            rows = torch.from_numpy(ctx_rows[r0:r0 + 4096]).to(t.key.device)
            key = W.bf16_as_f32_numpy(t.key.index_select(0, rows))
            value = W.bf16_as_f32_numpy(t.value.index_select(0, rows))
            sl = slots_all[ctx_rows[r0:r0 + 4096]]
            t0 = time.perf_counter()
            if mode == "int4":
                O.write_kv(key, value, sl, nb, w.block_size, w.sign_seed)
            else:
                O.pth_write_kv(key, value, sl, nb, w.block_size, mode)
            wr_spent += time.perf_counter() - t0
            wr_tok += len(sl)
            if wr_spent >= budget_s / 5:
                break
    res = {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
           "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
           "sample": f"attention: {done_seqs} of {w.num_seqs} sequences of {w.name} (fp64 numpy oracle reading "
                     f"the GPU-written cache), {spent:.1f} s of CPU time; write: {wr_tok} context tokens "
                     f"(spec-tier numpy oracle, K and V), {wr_spent:.1f} s",
           "attn_query_tokens_per_s": round(done_q / spent, 2),
           "numpy": np.__version__, "blas": blas}
    if wr_tok:
        res["write_tokens_per_s"] = round(wr_tok / wr_spent, 1)
    return res


if __name__ == "__main__":
    main()
