"""Shared plumbing for the GPU parity tests: run the HIP path through the
binding, and run the oracle on the same seeded inputs. Nothing here computes
any part of the method itself."""
from __future__ import annotations

import dataclasses
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_decode_attention_reshape_amd as kv4  # noqa: E402
import workloads as W  # noqa: E402
from oracle import kv4_oracle as O  # noqa: E402

DEV = torch.device("cuda:0")


def say(msg: str):
    print(msg, flush=True)


@dataclasses.dataclass
class GpuRun:
    w: W.Workload
    lay: W.Layout
    t: W.Tensors            # bf16 inputs (device of generation)
    slots: np.ndarray       # slot of every KV token (concatenated row order)
    kc: torch.Tensor
    vc: torch.Tensor
    ks: torch.Tensor
    vs: torch.Tensor
    out: torch.Tensor = None


def alloc_cache(w: W.Workload, num_blocks: int, fill: int = 0):
    kc = torch.full((num_blocks, w.block_size, w.num_kv_heads, w.head_size // 2), fill, dtype=torch.uint8,
                    device=DEV)
    vc = torch.full_like(kc, fill)
    ks = torch.full((num_blocks, w.block_size, w.num_kv_heads), float(fill), dtype=torch.float32, device=DEV)
    vs = torch.full_like(ks, float(fill))
    return kc, vc, ks, vs


def run_gpu(w: W.Workload, gen_device="cpu", attention=True, fill=0, softmax_scale=None,
            len_slack=(0, 0)) -> GpuRun:
    """Generate inputs, write every KV token with kv4_rht_write (one call),
    run kv4_paged_attention over the batch. len_slack adds to the host-side
    max_query_len / max_seq_len bounds (upper bounds need not be tight)."""
    say(f"[gpu] case {w.name}: nq={w.num_q_heads} nkv={w.num_kv_heads} hs={w.head_size} "
        f"bs={w.block_size} seqs={w.num_seqs} q_tokens={w.num_q_tokens} kv_tokens={w.total_kv_tokens}")
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay, device=gen_device)
    slots = W.all_slots(lay, w)
    kc, vc, ks, vs = alloc_cache(w, lay.num_blocks, fill)
    kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), kc, vc, ks, vs, torch.from_numpy(slots).to(DEV),
                      sign_seed=w.sign_seed)
    r = GpuRun(w, lay, t, slots, kc, vc, ks, vs)
    if attention:
        r.out = kv4.kv4_paged_attention(
            t.query.to(DEV), kc, vc, ks, vs, torch.from_numpy(lay.block_table).to(DEV),
            torch.from_numpy(lay.seq_lens).to(DEV), torch.from_numpy(lay.query_start_loc).to(DEV),
            max_query_len=w.max_query_len + len_slack[0], max_seq_len=w.max_seq_len + len_slack[1],
            sign_seed=w.sign_seed, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return r


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().numpy()


def oracle_attention_on_gpu_cache(r: GpuRun, seqs=None, softmax_scale=None) -> np.ndarray:
    """G2 reference: fp64 oracle reading the cache the GPU wrote."""
    w = r.w
    q = W.bf16_as_f32_numpy(r.t.query)
    sc = w.head_size ** -0.5 if softmax_scale is None else softmax_scale
    return O.paged_attention(q, host(r.kc), host(r.vc), host(r.ks), host(r.vs), r.lay.block_table,
                             r.lay.seq_lens, r.lay.query_start_loc, sc, w.sign_seed, seqs=seqs)


def oracle_caches(r: GpuRun):
    key, value = W.bf16_as_f32_numpy(r.t.key), W.bf16_as_f32_numpy(r.t.value)
    return O.write_kv(key, value, r.slots, r.lay.num_blocks, r.w.block_size, r.w.sign_seed)


def allclose_report(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float):
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    return int(bad.sum()), float(err.max()) if err.size else 0.0


def corr(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.corrcoef(a.ravel(), b.ravel())[0, 1])


def inline_rows(buf: np.ndarray, mode: str, nkv: int, hs: int, bs: int):
    """Vectorized reader of an inline-scale buffer (uint8 [nb, block_bytes]):
    (kc, vc, ks, vs) with the geometry the oracle defines (inline_geometry);
    the same result as O.inline_unpack, without its per-row Python loops, and
    the padding bytes of every row as a fifth value. Host logic only."""
    geo = O.inline_geometry(mode, nkv, hs, bs)
    c, pitch = geo["code_bytes"], geo["pitch"]
    rows = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1, 2, bs, nkv, pitch)
    codes = rows[..., :c]
    scales = np.ascontiguousarray(rows[..., c:c + 4]).view(np.float32)[..., 0]
    pad = rows[..., c + 4:]
    return (np.ascontiguousarray(codes[:, 0]), np.ascontiguousarray(codes[:, 1]),
            np.ascontiguousarray(scales[:, 0]), np.ascontiguousarray(scales[:, 1]), pad)


def worker_count() -> int:
    """CPU workers for oracle work: the host cores this process may use, at
    most 16 (a GPU machine's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))
