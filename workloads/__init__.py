"""Seeded synthetic inputs for the INT4 per-token-head KV-cache path.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It only draws random numbers and builds index structures (sequence
lengths, page tables, slot mappings, query offsets). It holds none of the
method's arithmetic: no rotation, no rounding of the rotated values, no
quantization, no attention.

Workload shapes follow the serving configurations discussed on the pages
(Phi-3-mini head_size 96 with non-power-of-two Hadamard blocks, Llama-3.2-1B,
Qwen2.5-1.5B and Llama-3-8B shaped GQA, paged KV with block_size 16), with
synthetic N(0, 1) bf16 tensors in place of model activations.

Recipe (stated once here, used everywhere):
  * sequence lengths, page permutations and outlier masks come from
    ``numpy.random.Generator(PCG64(seed))`` -- identical on every machine;
  * bulk tensors (Q, K, V) are N(0, 1) float32 draws from a seeded
    ``torch.Generator`` on the target device, cast to bf16 by torch
    (round-to-nearest-even). CPU and GPU generators give different streams,
    so a test that compares against the oracle either generates on the CPU
    or copies the sampled input rows back from the device;
  * outlier channels (Llama-3-8B long-context shape): one Bernoulli(0.01)
    mask per (kv head, channel), the same for every token, multiplies those
    K and V channels by 20 before the bf16 cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16
DEFAULT_SIGN_SEED = 42


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named batch shape: per sequence (query_len, seq_len)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    query_lens: tuple
    seq_lens: tuple
    shuffle_pages: bool = True
    shuffle_seqs: bool = False
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    sign_seed: int = DEFAULT_SIGN_SEED
    data_seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def num_q_tokens(self) -> int:
        return int(sum(self.query_lens))

    @property
    def max_query_len(self) -> int:
        return int(max(self.query_lens)) if self.query_lens else 0

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    @property
    def total_kv_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def b(self) -> int:
        return self.head_size & -self.head_size


def _loguniform_ints(rng: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    return np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)


def tiny(kv_len: int, seed: int = 0) -> Workload:
    """1 sequence, 4 q / 4 kv heads, head_size 128, one decode query."""
    return Workload(
        name=f"tiny_L{kv_len}", num_q_heads=4, num_kv_heads=4, head_size=128,
        block_size=BLOCK_SIZE, query_lens=(1,), seq_lens=(kv_len,),
        shuffle_pages=False, data_seed=seed)


def phi3(seed: int = 0, batch: int = 32, ctx: int = 1024) -> Workload:
    """Phi-3-mini shape: 32/32 heads, head_size 96 (b = 32), decode."""
    return Workload(
        name="phi3_hs96_b32x1024", num_q_heads=32, num_kv_heads=32, head_size=96,
        block_size=BLOCK_SIZE, query_lens=(1,) * batch, seq_lens=(ctx,) * batch,
        data_seed=seed)


def llama1b(seed: int = 0, batch: int = 64) -> Workload:
    """Llama-3.2-1B shape: 32/8 heads, head_size 64, ctx U[1024, 4096]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1024, 4096, size=batch, endpoint=True)
    return Workload(
        name="llama1b_hs64_b64", num_q_heads=32, num_kv_heads=8, head_size=64,
        block_size=BLOCK_SIZE, query_lens=(1,) * batch,
        seq_lens=tuple(int(x) for x in lens), data_seed=seed)


def qwen_mixed(seed: int = 0, n_prefill: int = 4, chunk: int = 512, prefix: int = 2048,
               n_decode: int = 60) -> Workload:
    """Qwen2.5-1.5B shape: 12/2 heads, head_size 128; chunked prefill + decode,
    sequences in shuffled order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dec = _loguniform_ints(rng, 256, 8192, n_decode)
    qlens = [chunk] * n_prefill + [1] * n_decode
    slens = [prefix + chunk] * n_prefill + [int(x) for x in dec]
    order = rng.permutation(len(qlens))
    return Workload(
        name="qwen1p5b_mixed", num_q_heads=12, num_kv_heads=2, head_size=128,
        block_size=BLOCK_SIZE, query_lens=tuple(qlens[i] for i in order),
        seq_lens=tuple(slens[i] for i in order), shuffle_seqs=True, data_seed=seed)


def qwen_prefill(seed: int = 0) -> Workload:
    """The chunked-prefill part of the Qwen2.5-1.5B mixed batch alone: its 4
    sequences of 512 new tokens on a 2048-token prefix, no decode sequences."""
    w = qwen_mixed(seed)
    keep = [i for i, q in enumerate(w.query_lens) if q > 1]
    return Workload(
        name="qwen1p5b_prefill4x512", num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
        head_size=w.head_size, block_size=w.block_size,
        query_lens=tuple(w.query_lens[i] for i in keep), seq_lens=tuple(w.seq_lens[i] for i in keep),
        shuffle_seqs=True, data_seed=seed)


def llama8b_long(seed: int = 0, batch: int = 128) -> Workload:
    """Llama-3-8B shape: 32/8 heads, head_size 128, ctx log-U[4096, 32768],
    1 % outlier channels x20."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = _loguniform_ints(rng, 4096, 32768, batch)
    return Workload(
        name="llama8b_hs128_b128_logU4k-32k", num_q_heads=32, num_kv_heads=8,
        head_size=128, block_size=BLOCK_SIZE, query_lens=(1,) * batch,
        seq_lens=tuple(int(x) for x in lens), outlier_frac=0.01, data_seed=seed)


def llama8b_spec(seed: int = 0, batch: int = 128, qmin: int = 2, qmax: int = 8) -> Workload:
    """Multi-token decode at the long-context Llama-3-8B shape: each sequence
    scores qmin..qmax new tokens at once (speculative-decode-like), ctx
    log-U[4096, 32768], 1 % outlier channels x20."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = _loguniform_ints(rng, 4096, 32768, batch)
    qlens = rng.integers(qmin, qmax, size=batch, endpoint=True)
    return Workload(
        name=f"llama8b_hs128_b{batch}_q{qmin}-{qmax}_logU4k-32k", num_q_heads=32, num_kv_heads=8,
        head_size=128, block_size=BLOCK_SIZE, query_lens=tuple(int(x) for x in qlens),
        seq_lens=tuple(int(x) for x in lens), outlier_frac=0.01, data_seed=seed)


def llama8b_hs192(seed: int = 0, batch: int = 32, ctx: int = 16384) -> Workload:
    """Secondary sweep of the long-context shape: head_size 192 (b = 64)."""
    return Workload(
        name="llama8b_hs192_b32x16k", num_q_heads=32, num_kv_heads=8, head_size=192,
        block_size=BLOCK_SIZE, query_lens=(1,) * batch, seq_lens=(ctx,) * batch,
        outlier_frac=0.01, data_seed=seed)


def hs256_long(seed: int = 0, batch: int = 128) -> Workload:
    """Head size 256 at the long-context batch: 16/4 heads (the same cache
    bytes per token as 32/8 heads of 128), ctx log-U[4096, 32768], 1 % outlier
    channels x20."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = _loguniform_ints(rng, 4096, 32768, batch)
    return Workload(
        name="gqa16x4_hs256_b128_logU4k-32k", num_q_heads=16, num_kv_heads=4,
        head_size=256, block_size=BLOCK_SIZE, query_lens=(1,) * batch,
        seq_lens=tuple(int(x) for x in lens), outlier_frac=0.01, data_seed=seed)


def custom(name: str, nq: int, nkv: int, hs: int, query_lens: Sequence[int],
           seq_lens: Sequence[int], block_size: int = BLOCK_SIZE, shuffle_pages: bool = True,
           seed: int = 0, sign_seed: int = DEFAULT_SIGN_SEED, outlier_frac: float = 0.0) -> Workload:
    return Workload(name=name, num_q_heads=nq, num_kv_heads=nkv, head_size=hs,
                    block_size=block_size, query_lens=tuple(int(x) for x in query_lens),
                    seq_lens=tuple(int(x) for x in seq_lens), shuffle_pages=shuffle_pages,
                    data_seed=seed, sign_seed=sign_seed, outlier_frac=outlier_frac)


@dataclasses.dataclass
class Layout:
    """Page tables and offsets for a workload (all numpy, host side)."""

    block_table: np.ndarray      # int32 [num_seqs, max_blocks_per_seq]
    seq_lens: np.ndarray         # int32 [num_seqs]
    query_start_loc: np.ndarray  # int32 [num_seqs + 1]
    num_blocks: int
    # token rows of the per-sequence K/V tensors, concatenated: sequence s owns
    # rows kv_start[s] .. kv_start[s] + seq_lens[s]
    kv_start: np.ndarray         # int64 [num_seqs + 1]


def make_layout(w: Workload) -> Layout:
    """Page tables: sequence s owns ceil(L_s / block_size) pages. With
    shuffle_pages the physical page ids are a random permutation (non-contiguous
    tables); one spare page is allocated and never referenced."""
    rng = np.random.Generator(np.random.PCG64(w.data_seed + 1_000_003))
    bs = w.block_size
    nblk = [(-(-L // bs)) for L in w.seq_lens]
    total = int(sum(nblk))
    num_blocks = total + 1
    ids = rng.permutation(num_blocks)[:total] if w.shuffle_pages else np.arange(total)
    maxb = max(nblk) if nblk else 1
    bt = np.zeros((w.num_seqs, max(maxb, 1)), dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        bt[s, :n] = ids[off:off + n]
        off += n
    qsl = np.zeros(w.num_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(w.query_lens)
    kvs = np.zeros(w.num_seqs + 1, dtype=np.int64)
    kvs[1:] = np.cumsum(w.seq_lens)
    return Layout(block_table=bt, seq_lens=np.asarray(w.seq_lens, dtype=np.int32),
                  query_start_loc=qsl, num_blocks=num_blocks, kv_start=kvs)


def slots_for(layout: Layout, w: Workload, seq: int, positions: np.ndarray) -> np.ndarray:
    """Physical slot ids of token positions of one sequence (page * bs + offset)."""
    positions = np.asarray(positions, dtype=np.int64)
    bs = w.block_size
    page = layout.block_table[seq, positions // bs].astype(np.int64)
    return page * bs + positions % bs


def all_slots(layout: Layout, w: Workload) -> np.ndarray:
    """Slot of every KV token, in the concatenated (sequence-major) row order."""
    out = np.empty(int(layout.kv_start[-1]), dtype=np.int64)
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        out[layout.kv_start[s]:layout.kv_start[s] + L] = slots_for(layout, w, s, np.arange(L))
    return out


def new_token_rows(layout: Layout, w: Workload) -> np.ndarray:
    """Rows (in concatenated KV order) of the tokens written in the step: the
    last query_len positions of every sequence."""
    rows = []
    for s in range(w.num_seqs):
        L, q = int(w.seq_lens[s]), int(w.query_lens[s])
        rows.append(np.arange(layout.kv_start[s] + L - q, layout.kv_start[s] + L))
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def outlier_mask(w: Workload) -> Optional[np.ndarray]:
    """[num_kv_heads, head_size] float32 channel gains (1 or outlier_gain)."""
    if w.outlier_frac <= 0:
        return None
    rng = np.random.Generator(np.random.PCG64(w.data_seed + 2_000_029))
    m = rng.random((w.num_kv_heads, w.head_size)) < w.outlier_frac
    return np.where(m, np.float32(w.outlier_gain), np.float32(1.0)).astype(np.float32)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal_bf16(shape, seed: int, device="cpu", gain: Optional[np.ndarray] = None,
                chunk_rows: int = 1 << 18) -> torch.Tensor:
    """N(0, 1) float32 draws cast to bf16, generated in row chunks on `device`.
    `gain` (broadcast over the trailing dims) multiplies before the cast."""
    shape = tuple(int(x) for x in shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if shape[0] == 0:
        return out
    g = _generator(device, seed)
    gt = None if gain is None else torch.from_numpy(gain).to(device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0,) + shape[1:], generator=g, dtype=torch.float32, device=device)
        if gt is not None:
            x = x * gt
        out[r0:r1] = x.to(torch.bfloat16)
    return out


@dataclasses.dataclass
class Tensors:
    key: torch.Tensor     # bf16 [total_kv_tokens, nkv, hs]
    value: torch.Tensor   # bf16 [total_kv_tokens, nkv, hs]
    query: torch.Tensor   # bf16 [num_q_tokens, nq, hs]


def make_tensors(w: Workload, layout: Layout, device="cpu") -> Tensors:
    gain = outlier_mask(w)
    T = int(layout.kv_start[-1])
    base = w.data_seed * 1_000_000_007
    key = normal_bf16((T, w.num_kv_heads, w.head_size), base + 11, device, gain)
    value = normal_bf16((T, w.num_kv_heads, w.head_size), base + 13, device, gain)
    query = normal_bf16((w.num_q_tokens, w.num_q_heads, w.head_size), base + 17, device)
    return Tensors(key=key, value=value, query=query)


def bf16_as_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact float32 values of a bf16 tensor, as a host numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy()


ALL = {
    "tiny32": lambda: tiny(32),
    "tiny64": lambda: tiny(64),
    "tiny128": lambda: tiny(128),
    "phi3": phi3,
    "llama1b": llama1b,
    "qwen_mixed": qwen_mixed,
    "qwen_prefill": qwen_prefill,
    "llama8b_long": llama8b_long,
    "llama8b_hs192": llama8b_hs192,
    "hs256_long": hs256_long,
    "llama8b_spec": llama8b_spec,
    "llama8b_spec4": lambda: llama8b_spec(qmin=4, qmax=4),
}
