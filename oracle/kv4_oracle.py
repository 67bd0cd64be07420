"""CPU oracle for the INT4 per-token-head RHT KV cache (write + paged attention).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU product path never calls it,
and it shares no code, tables or constants with the HIP sources.

Sources (cited by title and section):
  [PR40835]  vLLM PR #40835, "[Feature] Triton INT4 per-token-head KV cache
             quantization" -- review thread (scale-cache shapes, uint8 cache,
             slot mapping, query_start_loc / seq_lens metadata).
  [PR56198]  runguoli.com, "vLLM -- Attention Kernels & KV Cache Quantization",
             section "PR #56198 -- Support int4_per_token_head on
             non-power-of-two head sizes" (block-diagonal H_b, b = largest
             power-of-two divisor, compensation by b, fp64 reference errors).
  [PR62881]  vLLM PR #62881, "[Bugfix][Test] Rotate KV into RHT domain in the
             INT4 unified attn test" -- Details: Root cause (K_s = H.D.k,
             q' = H.D.q with softmax_scale / d, output D.H(.)/d), Fix (rotation
             rounded through bf16 before quantizing), Tolerance.

Two tiers:
  * spec tier  -- the exact float32 / bf16 operation order the write path is
                  defined with (radix-2 butterflies in ascending stride order,
                  one round-to-nearest-even to bf16, IEEE float32 division).
                  Used for bit-exact comparison of codes and scales.
  * math tier  -- fp64: explicit dense block-diagonal Hadamard matrix,
                  scalar quantization, unpaged attention.

Readings where the pages are silent:
  D: sign i is -1 iff bit 63 of the (i+1)-th SplitMix64 output seeded with
     sign_seed is set; one D of length head_size shared by K, V, Q, all heads
     and tokens.  H_b: Sylvester order, entry (r, c) = (-1)^popcount(r & c),
     unnormalized.  Blocks are contiguous chunks [j*b, (j+1)*b).  The int4 rule
     is absmax / 7, round-half-to-even of the float32 quotient, clamp [-8, 7],
     two's-complement nibbles, element 2j in the low nibble of byte j.  amax == 0
     stores scale 0 and codes 0.  A slot outside [0, num_blocks * block_size)
     skips the token.  Query i of a
     sequence with query_len q and seq_len L sits at position L - q + i and
     attends to keys 0..L-q+i.
"""
from __future__ import annotations

import numpy as np

_M64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


# ---------------------------------------------------------------------------
# Randomized signs D and the block-diagonal Hadamard H  ([PR56198], [PR62881])
# ---------------------------------------------------------------------------

def splitmix64(seed: int, n: int) -> list:
    """First n outputs of SplitMix64 (Steele, Lea & Flood 2014, as published in
    Vigna's public-domain splitmix64.c) started from state `seed`. Plain Python
    integers, one output at a time."""
    x = seed & _M64
    out = []
    for _ in range(n):
        x = (x + _GOLDEN_GAMMA) & _M64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def rht_signs(sign_seed: int, head_size: int) -> np.ndarray:
    """Diagonal of D (float64 +-1): D.D = I ([PR62881] Root cause)."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(sign_seed, head_size)])


def largest_pow2_divisor(n: int) -> int:
    """b: the largest power of two dividing head_size ([PR56198])."""
    if n <= 0:
        raise ValueError("head_size must be positive")
    b = 1
    while n % (2 * b) == 0:
        b *= 2
    return b


def hadamard(b: int) -> np.ndarray:
    """Unnormalized Sylvester Hadamard H_b, entries (-1)^popcount(r & c)."""
    if b <= 0 or (b & (b - 1)):
        raise ValueError("b must be a power of two")
    H = np.empty((b, b), dtype=np.float64)
    for r in range(b):
        for c in range(b):
            H[r, c] = -1.0 if bin(r & c).count("1") % 2 else 1.0
    return H


def block_diag_hadamard(head_size: int) -> np.ndarray:
    """H for head_size d = b * n: H_b repeated n times on the diagonal
    ([PR56198]: H @ H.T = b * I, no padding)."""
    b = largest_pow2_divisor(head_size)
    Hb = hadamard(b)
    H = np.zeros((head_size, head_size), dtype=np.float64)
    for j in range(head_size // b):
        H[j * b:(j + 1) * b, j * b:(j + 1) * b] = Hb
    return H


def rotate_math(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp64 H . D . x along the last axis ([PR62881] Root cause: K_s = H.D.k)."""
    H = block_diag_hadamard(x.shape[-1])
    return (np.asarray(x, dtype=np.float64) * signs) @ H.T


def unrotate_math(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp64 D . H . y / b along the last axis: the inverse of rotate_math
    ([PR62881] Root cause, output compensation; divisor b per [PR56198])."""
    d = y.shape[-1]
    H = block_diag_hadamard(d)
    return (np.asarray(y, dtype=np.float64) @ H.T) * signs / largest_pow2_divisor(d)


# ---------------------------------------------------------------------------
# Spec tier of the write path (float32 / bf16, fixed operation order)
# ---------------------------------------------------------------------------

def fwht_spec_f32(x: np.ndarray, b: int) -> np.ndarray:
    """Radix-2 fast Walsh-Hadamard transform of every contiguous b-chunk of the
    last axis, in float32: for stride h = 1, 2, 4, ..., b/2 and every index i
    with (i & h) == 0 inside a chunk, (x_i, x_{i+h}) <- (x_i + x_{i+h},
    x_i - x_{i+h}), each one IEEE float32 operation. Same matrix as hadamard(b)
    (Sylvester order)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d % b:
        raise ValueError("b must divide the last axis")
    v = y.reshape(y.shape[:-1] + (d // b, b))
    h = 1
    while h < b:
        w = v.reshape(v.shape[:-1] + (b // (2 * h), 2, h))
        lo = w[..., 0, :].copy()
        hi = w[..., 1, :].copy()
        w[..., 0, :] = lo + hi
        w[..., 1, :] = lo - hi
        h *= 2
    return v.reshape(y.shape)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as the
    exact float32 value of that bf16. Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def rotate_spec(x_bf16: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """The stored rotation of one head vector: sign flip (exact), float32
    block butterflies, one bf16 rounding ([PR62881] Fix: rotation rounded
    through bf16 before quantizing)."""
    d = x_bf16.shape[-1]
    xs = np.asarray(x_bf16, dtype=np.float32) * signs.astype(np.float32)
    return bf16_round(fwht_spec_f32(xs, largest_pow2_divisor(d)))


def quantize_int4(y: np.ndarray):
    """Per-(token, head) symmetric int4: scale = float32(absmax) / 7 (IEEE
    float32 division), code = clamp(rint_half_even(float32(y / scale)), -8, 7).
    amax == 0 gives scale 0 and all-zero codes. One fp32 scale per vector
    ([PR40835] review: scale caches are float32 per (token, kv head))."""
    y = np.asarray(y, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1)
    scale = (amax / np.float32(7.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (y / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(q), -8, 7).astype(np.int8)
    codes = np.where(scale[..., None] > 0, codes, np.int8(0)).astype(np.int8)
    return codes, scale


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2j in the low nibble of byte j."""
    c = np.asarray(codes, dtype=np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# Paged cache (write, gather, dequant)
# ---------------------------------------------------------------------------

def new_cache(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    """Zeroed uint8 [nb, bs, nkv, hs/2] codes and float32 [nb, bs, nkv] scales
    ([PR40835] review: uint8 int4 cache, float32 scale caches)."""
    codes = np.zeros((num_blocks, block_size, num_kv_heads, head_size // 2), dtype=np.uint8)
    scales = np.zeros((num_blocks, block_size, num_kv_heads), dtype=np.float32)
    return codes, scales


def rht_write(x_bf16: np.ndarray, cache: np.ndarray, scale_cache: np.ndarray,
              slot_mapping: np.ndarray, sign_seed: int, chunk: int = 16384) -> None:
    """Write path for one of K or V: rotate, round through bf16, quantize and
    pack each (token, kv head) vector into its slot (blk = slot // bs,
    off = slot % bs; [PR40835] review round-trip loop). Slots outside
    [0, num_blocks * bs) name no cache row and are skipped. Every vector is
    independent; tokens are processed a chunk at a time."""
    x = np.asarray(x_bf16, dtype=np.float32)
    T, nkv, hs = x.shape
    bs = cache.shape[1]
    signs = rht_signs(sign_seed, hs)
    sl = np.asarray(slot_mapping, dtype=np.int64)
    for t0 in range(0, T, chunk):
        s = sl[t0:t0 + chunk]
        keep = (s >= 0) & (s < cache.shape[0] * bs)
        if not keep.any():
            continue
        y = rotate_spec(x[t0:t0 + chunk][keep], signs)      # [t, nkv, hs]
        codes, scale = quantize_int4(y)
        s = s[keep]
        cache[s // bs, s % bs] = pack_int4(codes)
        scale_cache[s // bs, s % bs] = scale


def write_kv(key, value, slot_mapping, num_blocks, block_size, sign_seed):
    """Convenience: fresh caches with every token of key/value written."""
    T, nkv, hs = np.asarray(key).shape
    kc, ks = new_cache(num_blocks, block_size, nkv, hs)
    vc, vs = new_cache(num_blocks, block_size, nkv, hs)
    rht_write(key, kc, ks, slot_mapping, sign_seed)
    rht_write(value, vc, vs, slot_mapping, sign_seed)
    return kc, vc, ks, vs


def dequant(cache: np.ndarray, scale_cache: np.ndarray, slot_mapping: np.ndarray,
            sign_seed: int, inverse_rotate: bool) -> np.ndarray:
    """Gather slots and dequantize: code * scale as one float32 product; with
    inverse_rotate, D.H(.)/b in fp64 back to the original domain."""
    bs = cache.shape[1]
    sl = np.asarray(slot_mapping, dtype=np.int64)
    codes = unpack_int4(cache[sl // bs, sl % bs]).astype(np.float32)
    sc = scale_cache[sl // bs, sl % bs].astype(np.float32)
    y = (codes * sc[..., None]).astype(np.float32)
    if not inverse_rotate:
        return y
    signs = rht_signs(sign_seed, cache.shape[-1] * 2)
    return unrotate_math(y.astype(np.float64), signs)


def gather_seq(cache: np.ndarray, scale_cache: np.ndarray, block_table_row: np.ndarray,
               seq_len: int) -> np.ndarray:
    """fp64 dequantized [seq_len, nkv, hs] of one sequence, read through its
    page table (rotated domain)."""
    bs = cache.shape[1]
    pos = np.arange(seq_len)
    blk = np.asarray(block_table_row, dtype=np.int64)[pos // bs]
    off = pos % bs
    codes = unpack_int4(cache[blk, off]).astype(np.float64)
    return codes * scale_cache[blk, off].astype(np.float64)[..., None]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _causal_softmax_attend(logits: np.ndarray, vals: np.ndarray, L: int, window: int = 0) -> np.ndarray:
    """logits [ql, ..., L]: row i (query i of ql, position pos = L - ql + i)
    may see keys 0 .. pos, and with a sliding window W > 0 only keys j with
    pos - W < j <= pos (the W most recent); returns softmax(logits) @ vals
    with vals [L, hs]. A row that sees no key at all (pos < 0: the sequence
    is shorter than its query block) is exactly 0 -- the reading taken for
    an empty causal window, where the softmax has no terms."""
    ql = logits.shape[0]
    hs = vals.shape[-1]
    pos = L - ql + np.arange(ql)
    keys = np.arange(L)[None, :]
    mask = keys > pos[:, None]                                    # [ql, L]
    if window > 0:
        mask |= keys <= pos[:, None] - window
    empty = mask.all(axis=-1)                                     # [ql]; all True when L == 0
    if empty.all():
        return np.zeros(logits.shape[:-1] + (hs,))
    mask = mask.reshape((ql,) + (1,) * (logits.ndim - 2) + (L,))
    # an empty row gets one unmasked key for the arithmetic and is zeroed below
    mask = mask & ~empty.reshape((ql,) + (1,) * (logits.ndim - 1))
    lg = np.where(mask, -np.inf, logits)
    m = lg.max(axis=-1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=-1, keepdims=True)
    out = p @ vals
    out[empty] = 0.0
    return out


def paged_attention(query, key_cache, value_cache, k_scale_cache, v_scale_cache,
                    block_table, seq_lens, query_start_loc, softmax_scale: float,
                    sign_seed: int, seqs=None, window: int = 0) -> np.ndarray:
    """fp64 attention over the int4 RHT cache in the rotated domain
    ([PR62881] Root cause; divisor b per [PR56198]):
        q' = H.D.q,  logit_j = (q' . K_s_j) * softmax_scale / b,
        o' = softmax(logit) @ V_s,  o = D.H.o' / b.
    K_s, V_s are the dequantized cache values gathered through block_table.
    Causal: query i of sequence s (query_len q, seq_len L) sees keys
    0 .. L - q + i; with window > 0 only the `window` most recent of them
    (the pages' "added window" commit names the feature and nothing more;
    reading: key j is visible iff pos - window < j <= pos). GQA: q head h
    reads kv head h // (nq / nkv).
    Returns fp64 [num_q_tokens, nq, hs]; rows of sequences not in `seqs`
    are NaN."""
    q = np.asarray(query, dtype=np.float64)
    Tq, nq, hs = q.shape
    nkv = key_cache.shape[2]
    group = nq // nkv
    b = largest_pow2_divisor(hs)
    signs = rht_signs(sign_seed, hs)
    out = np.full((Tq, nq, hs), np.nan)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if seqs is None:
        seqs = range(len(seq_lens))
    for s in seqs:
        L = int(seq_lens[s])
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        if q1 == q0:
            continue
        Ks = gather_seq(key_cache, k_scale_cache, block_table[s], L)     # [L, nkv, hs]
        Vs = gather_seq(value_cache, v_scale_cache, block_table[s], L)
        qr = rotate_math(q[q0:q1], signs)                                 # [ql, nq, hs]
        for g in range(nkv):
            qg = qr[:, g * group:(g + 1) * group, :]                      # [ql, group, hs]
            logits = (qg @ Ks[:, g, :].T) * softmax_scale / b            # [ql, group, L]
            o_rot = _causal_softmax_attend(logits, Vs[:, g, :], L, window)   # [ql, group, hs]
            out[q0:q1, g * group:(g + 1) * group] = unrotate_math(o_rot, signs)
    return out


def attention_dense(query, key, value, query_start_loc, seq_lens, softmax_scale: float,
                    kv_start, seqs=None, window: int = 0) -> np.ndarray:
    """Plain fp64 causal attention in the original domain:
    softmax(q . k * softmax_scale) @ v per sequence, GQA head h -> h // group.
    Rows of sequence s in `key`/`value` are kv_start[s] .. kv_start[s] + L_s.
    Used on unquantized K/V and on dequantized, inverse-rotated K/V."""
    q = np.asarray(query, dtype=np.float64)
    Tq, nq, hs = q.shape
    nkv = np.asarray(key).shape[1]
    group = nq // nkv
    out = np.full((Tq, nq, hs), np.nan)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if seqs is None:
        seqs = range(len(seq_lens))
    for s in seqs:
        L = int(seq_lens[s])
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        if q1 == q0:
            continue
        k0 = int(kv_start[s])
        k = np.asarray(key[k0:k0 + L], dtype=np.float64)
        v = np.asarray(value[k0:k0 + L], dtype=np.float64)
        for g in range(nkv):
            qg = q[q0:q1, g * group:(g + 1) * group, :]
            logits = (qg @ k[:, g, :].T) * softmax_scale
            out[q0:q1, g * group:(g + 1) * group] = _causal_softmax_attend(logits, v[:, g, :], L, window)
    return out


# ---------------------------------------------------------------------------
# Per-token-head INT8 / FP8 control modes (no rotation)
# ---------------------------------------------------------------------------
# The pages name int8_per_token_head and fp8_per_token_head as the control
# modes of the same kernels ([PR56198]: they never use the transform; [PR40835]
# review: int8 or FP8 cache dtype, float32 scale caches per (token, kv head)).
# Readings (the pages are silent on the rule): symmetric
# absmax per (token, kv head) vector, scale = float32(absmax) / qmax (IEEE
# float32 division) with qmax = 127 (int8) or 448 (the largest finite OCP
# e4m3fn value); int8 code = clamp(rint_half_even(float32(x / scale)), -128,
# 127); fp8 code = float32(x / scale) rounded to nearest-even e4m3fn,
# saturating at +-448; amax == 0 stores scale 0 and code 0. One code byte per
# element: cache uint8 [nb, bs, nkv, hs].

PTH_QMAX = {"int8": 127.0, "fp8": 448.0}


def fp8_e4m3fn_decode(codes) -> np.ndarray:
    """float64 value of OCP FP8 E4M3 (e4m3fn) bytes: sign bit 7, exponent bits
    6..3 (bias 7), mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6);
    S.1111.111 is NaN and there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3fn_encode(x) -> np.ndarray:
    """Round float32 values to the nearest e4m3fn value (ties to even mantissa),
    saturating magnitudes above 448 to 448; the sign bit follows the input's
    (-0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)     # exact
    neg = np.signbit(x)
    a = np.abs(x)
    # quantum of the binade holding a: 2^(e - 3) for normal e >= -6, 2^-9 below
    _, ex = np.frexp(np.where(a > 0, a, 1.0))                  # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.exp2(e - 3.0)
    mq = np.rint(a / quantum)                                   # half to even; exact division by 2^k
    # mq in [0, 16]: 16 moves to the next binade (mantissa 0)
    val = mq * quantum
    code_mag = np.zeros(a.shape, dtype=np.int64)
    sub = val < 2.0 ** -6
    code_mag = np.where(sub, (val / 2.0 ** -9).astype(np.int64), code_mag)
    _, ev = np.frexp(np.where(val > 0, val, 1.0))
    ev = ev - 1
    mant = np.where(val > 0, val / np.exp2(ev.astype(np.float64)) - 1.0, 0.0)   # exact, multiple of 1/8
    normal_code = ((ev + 7) << 3) | np.rint(mant * 8.0).astype(np.int64)
    code_mag = np.where(sub, code_mag, normal_code)
    code_mag = np.where(val >= 448.0, 0x7E, code_mag)          # saturate (0x7F is NaN)
    return (code_mag | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_pth(x: np.ndarray, mode: str):
    """Per-(token, head) symmetric int8 / fp8 of float32 vectors along the last
    axis: returns (uint8 codes, float32 scales). See the readings above."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(PTH_QMAX[mode])).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (x / safe[..., None]).astype(np.float32)
    if mode == "int8":
        codes = np.clip(np.rint(q), -128, 127).astype(np.int8).view(np.uint8)
    else:
        codes = fp8_e4m3fn_encode(q)
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def decode_pth(codes, mode: str) -> np.ndarray:
    """float64 values of stored int8 / fp8 code bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    if mode == "int8":
        return c.view(np.int8).astype(np.float64)
    return fp8_e4m3fn_decode(c)


def pth_new_cache(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    """Zeroed uint8 [nb, bs, nkv, hs] codes and float32 [nb, bs, nkv] scales."""
    codes = np.zeros((num_blocks, block_size, num_kv_heads, head_size), dtype=np.uint8)
    scales = np.zeros((num_blocks, block_size, num_kv_heads), dtype=np.float32)
    return codes, scales


def pth_write(x_bf16: np.ndarray, cache: np.ndarray, scale_cache: np.ndarray,
              slot_mapping: np.ndarray, mode: str) -> None:
    """Write path of the int8 / fp8 modes for one of K or V: quantize each
    (token, kv head) vector of the bf16 input (exactly float32) and store it
    at its slot; slots outside [0, nb * bs) are skipped."""
    x = np.asarray(x_bf16, dtype=np.float32)
    bs = cache.shape[1]
    s = np.asarray(slot_mapping, dtype=np.int64)
    keep = (s >= 0) & (s < cache.shape[0] * bs)
    if not keep.any():
        return
    codes, scale = quantize_pth(x[keep], mode)
    s = s[keep]
    cache[s // bs, s % bs] = codes
    scale_cache[s // bs, s % bs] = scale


def pth_write_kv(key, value, slot_mapping, num_blocks, block_size, mode: str):
    """Convenience: fresh int8 / fp8 caches with every token written."""
    T, nkv, hs = np.asarray(key).shape
    kc, ks = pth_new_cache(num_blocks, block_size, nkv, hs)
    vc, vs = pth_new_cache(num_blocks, block_size, nkv, hs)
    pth_write(key, kc, ks, slot_mapping, mode)
    pth_write(value, vc, vs, slot_mapping, mode)
    return kc, vc, ks, vs


def pth_dequant(cache: np.ndarray, scale_cache: np.ndarray, slot_mapping: np.ndarray,
                mode: str) -> np.ndarray:
    """Gather slots and dequantize: code value * scale as one float32 product."""
    bs = cache.shape[1]
    sl = np.asarray(slot_mapping, dtype=np.int64)
    vals = decode_pth(cache[sl // bs, sl % bs], mode).astype(np.float32)
    sc = scale_cache[sl // bs, sl % bs].astype(np.float32)
    return (vals * sc[..., None]).astype(np.float32)


def pth_gather_seq(cache, scale_cache, block_table_row, seq_len: int, mode: str) -> np.ndarray:
    """fp64 dequantized [seq_len, nkv, hs] of one sequence through its page table."""
    bs = cache.shape[1]
    pos = np.arange(seq_len)
    blk = np.asarray(block_table_row, dtype=np.int64)[pos // bs]
    off = pos % bs
    return decode_pth(cache[blk, off], mode) * scale_cache[blk, off].astype(np.float64)[..., None]


def pth_paged_attention(query, key_cache, value_cache, k_scale_cache, v_scale_cache,
                        block_table, seq_lens, query_start_loc, softmax_scale: float,
                        mode: str, seqs=None, window: int = 0) -> np.ndarray:
    """fp64 causal paged attention over an int8 / fp8 per-token-head cache, in
    the original domain: logit_j = (q . K_j) * softmax_scale with K_j, V_j the
    dequantized cache rows; same causal rule and GQA mapping as
    paged_attention. Rows of sequences not in `seqs` are NaN."""
    q = np.asarray(query, dtype=np.float64)
    Tq, nq, hs = q.shape
    nkv = key_cache.shape[2]
    group = nq // nkv
    out = np.full((Tq, nq, hs), np.nan)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if seqs is None:
        seqs = range(len(seq_lens))
    for s in seqs:
        L = int(seq_lens[s])
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        if q1 == q0:
            continue
        K = pth_gather_seq(key_cache, k_scale_cache, block_table[s], L, mode)
        V = pth_gather_seq(value_cache, v_scale_cache, block_table[s], L, mode)
        for g in range(nkv):
            qg = q[q0:q1, g * group:(g + 1) * group, :]
            logits = (qg @ K[:, g, :].T) * softmax_scale
            out[q0:q1, g * group:(g + 1) * group] = _causal_softmax_attend(logits, V[:, g, :], L, window)
    return out


# ---------------------------------------------------------------------------
# Inline-scale padded-slot cache layout  ([PR40835] review of
# `_ensure_scale_caches`; vLLM PR #62113 "16-byte-align per-token-head KV
# slots so Triton vectorizes loads")
# ---------------------------------------------------------------------------
# The review shows float32 views into the cache with
#   full_block_f32 = 2 * kv_half_bytes / 4,  slot_f32 = nkv * padded_hs * dtype_sz / 4,
#   head_f32 = padded_hs * dtype_sz / 4,    scale_off_f32 = hs * dtype_sz / 4,
# K scales in kv half 0 and V scales offset by kv_half_bytes. Reading (the
# pages give no more): one buffer per layer, a page is the K half then the V
# half, each half bs * nkv rows (slot-major, then head); a row is the C code
# bytes (C = hs / 2 for int4, hs for int8 / fp8; "hs * dtype_sz" above), the
# float32 scale right after them, then zero padding to a 16-byte pitch
# (padded_hs * dtype_sz = round_up(C + 4, 16)).

def inline_geometry(mode: str, nkv: int, hs: int, bs: int) -> dict:
    """Byte and float32-view sizes of the inline layout (see above)."""
    c = hs // 2 if mode == "int4" else hs
    pitch = -(-(c + 4) // 16) * 16
    kv_half = bs * nkv * pitch
    return {"code_bytes": c, "pitch": pitch, "kv_half_bytes": kv_half, "block_bytes": 2 * kv_half,
            "full_block_f32": 2 * kv_half // 4, "slot_f32": nkv * pitch // 4, "head_f32": pitch // 4,
            "scale_off_f32": c // 4}


def inline_row_offset(geo: dict, page: int, half: int, slot: int, head: int, nkv: int) -> int:
    """Byte offset of the row of (page, kv half 0 = K / 1 = V, slot, kv head)."""
    return page * geo["block_bytes"] + half * geo["kv_half_bytes"] + (slot * nkv + head) * geo["pitch"]


def inline_pack(kc, vc, ks, vs, mode: str) -> np.ndarray:
    """Packed caches (codes [nb, bs, nkv, C], float32 scales [nb, bs, nkv])
    -> the inline buffer uint8 [nb, block_bytes], padding zero. Python loops:
    small inputs only."""
    nb, bs, nkv, c = kc.shape
    hs = 2 * c if mode == "int4" else c
    geo = inline_geometry(mode, nkv, hs, bs)
    buf = np.zeros(nb * geo["block_bytes"], dtype=np.uint8)
    for p in range(nb):
        for half, (codes, sc) in enumerate(((kc, ks), (vc, vs))):
            for t in range(bs):
                for h in range(nkv):
                    o = inline_row_offset(geo, p, half, t, h, nkv)
                    buf[o:o + c] = codes[p, t, h]
                    buf[o + c:o + c + 4] = np.frombuffer(np.float32(sc[p, t, h]).tobytes(), dtype=np.uint8)
    return buf.reshape(nb, geo["block_bytes"])


def inline_unpack(buf, mode: str, nkv: int, hs: int, bs: int):
    """Inverse of inline_pack: (kc, vc, ks, vs) from the inline buffer."""
    geo = inline_geometry(mode, nkv, hs, bs)
    flat = np.asarray(buf, dtype=np.uint8).reshape(-1)
    nb = flat.size // geo["block_bytes"]
    c = geo["code_bytes"]
    kc = np.zeros((nb, bs, nkv, c), dtype=np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((nb, bs, nkv), dtype=np.float32)
    vs = np.zeros_like(ks)
    for p in range(nb):
        for half, (codes, sc) in enumerate(((kc, ks), (vc, vs))):
            for t in range(bs):
                for h in range(nkv):
                    o = inline_row_offset(geo, p, half, t, h, nkv)
                    codes[p, t, h] = flat[o:o + c]
                    sc[p, t, h] = flat[o + c:o + c + 4].view(np.float32)[0]
    return kc, vc, ks, vs


def inline_store_rows(buf, kc, vc, ks, vs, slot_mapping, mode: str) -> None:
    """The inline layout's write: copy the rows of the given slots (from the
    packed caches the write path computed) into an existing inline buffer;
    padding and other rows keep their bytes. Slots outside the cache are
    skipped."""
    nb, bs, nkv, c = kc.shape
    hs = 2 * c if mode == "int4" else c
    geo = inline_geometry(mode, nkv, hs, bs)
    flat = buf.reshape(-1)
    for s in np.asarray(slot_mapping, dtype=np.int64):
        if s < 0 or s >= nb * bs:
            continue
        p, t = int(s // bs), int(s % bs)
        for half, (codes, sc) in enumerate(((kc, ks), (vc, vs))):
            for h in range(nkv):
                o = inline_row_offset(geo, p, half, t, h, nkv)
                flat[o:o + c] = codes[p, t, h]
                flat[o + c:o + c + 4] = np.frombuffer(np.float32(sc[p, t, h]).tobytes(), dtype=np.uint8)
