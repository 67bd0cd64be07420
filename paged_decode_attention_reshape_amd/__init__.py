"""Python binding of libkv4 (INT4 per-token-head RHT KV cache on MI355X).

Argument marshalling only: every step of the write path, the paged attention
and the dequant helper runs in the HIP kernels of libkv4.so (see
include/kv4.h for the C contracts). torch supplies device memory and the
current HIP stream. The functions keep the C names.

The library must have been built (``python -m
paged_decode_attention_reshape_amd.build`` or ``__graft_entry__.build()``);
importing the functions without it raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KV4_LIBRARY selects another build of the same ABI (e.g. libkv4_debug.so)
LIB_PATH = os.environ.get("KV4_LIBRARY") or os.path.join(_HERE, "libkv4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kv4.h")

KV4_OK, KV4_EINVAL, KV4_EUNSUPPORTED, KV4_EHIP, KV4_EWORKSPACE = 0, 1, 2, 3, 4
KV4_MODE_INT8, KV4_MODE_FP8 = 1, 2
_MODES = {"int8": KV4_MODE_INT8, "fp8": KV4_MODE_FP8, KV4_MODE_INT8: KV4_MODE_INT8, KV4_MODE_FP8: KV4_MODE_FP8}
DEFAULT_SIGN_SEED = 42

_c_int32, _c_int64, _c_uint64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p


class CacheLayout(ctypes.Structure):
    """kv4_cache_layout: code strides in bytes, scale strides in floats."""
    _fields_ = [("block_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("scale_block_stride", ctypes.c_int64),
                ("scale_token_stride", ctypes.c_int64), ("scale_head_stride", ctypes.c_int64)]

    def as_tuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)


_LP = ctypes.POINTER(CacheLayout)
_SIGNATURES = {
    "kv4_rht_write": (ctypes.c_int, [_vp, _vp, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _vp, _c_int64,
                                     _c_int32, _c_int32, _c_int32, _c_int32, _c_int64, _c_uint64, _vp]),
    "kv4_paged_attention_workspace_size": (ctypes.c_size_t, [_c_int64, _c_int32, _c_int32, _c_int32,
                                                             _c_int32, _c_int32, _c_int32]),
    "kv4_paged_attention": (ctypes.c_int, [_vp, _c_int64, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int32,
                                           _vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32, _c_int32,
                                           _c_int32, _c_int32, _c_int32, _c_int32, _c_uint64,
                                           ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "kv4_paged_attention_noalloc": (ctypes.c_int, [_vp, _c_int64, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int32,
                                                   _vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32, _c_int32,
                                                   _c_int32, _c_int32, _c_int32, _c_int32, _c_uint64,
                                                   ctypes.c_float, _vp, _vp]),
    "kv4_dequant": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _c_int64, _c_int32, _c_int32, _c_int32,
                                   _c_int32, _c_uint64, _c_int32, _vp, _vp]),
    "kv4_last_error": (ctypes.c_char_p, []),
    "kv4_stream_read": (ctypes.c_int, [_vp, _c_int64, _vp, _c_int32, _vp]),
    "kv4_debug_flags": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), _c_int32]),
    "kv4_pth_write": (ctypes.c_int, [_c_int32, _vp, _vp, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _vp,
                                     _c_int64, _c_int32, _c_int32, _c_int32, _c_int64, _vp]),
    "kv4_pth_dequant": (ctypes.c_int, [_c_int32, _vp, _vp, _c_int64, _vp, _c_int64, _c_int32, _c_int32,
                                       _c_int32, _vp, _vp]),
    "kv4_pth_attention_workspace_size": (ctypes.c_size_t, [_c_int32, _c_int64, _c_int32, _c_int32, _c_int32,
                                                           _c_int32, _c_int32, _c_int32]),
    "kv4_pth_attention": (ctypes.c_int, [_c_int32, _vp, _c_int64, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int32,
                                         _vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32, _c_int32, _c_int32,
                                         _c_int32, _c_int32, ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "kv4_cache_layout_packed": (ctypes.c_int, [_c_int32, _c_int32, _c_int32, _c_int32, _LP]),
    "kv4_cache_layout_inline": (ctypes.c_int, [_c_int32, _c_int32, _c_int32, _c_int32, _LP,
                                               ctypes.POINTER(_c_int64), ctypes.POINTER(_c_int64),
                                               ctypes.POINTER(_c_int64)]),
    "kv4_write_layout": (ctypes.c_int, [_c_int32, _vp, _vp, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _LP, _vp,
                                        _c_int64, _c_int32, _c_int32, _c_int32, _c_int32, _c_int64, _c_uint64,
                                        _vp]),
    "kv4_attention_layout_workspace_size": (ctypes.c_size_t, [_c_int32, _LP, _c_int64, _c_int32, _c_int32,
                                                              _c_int32, _c_int32, _c_int32, _c_int32]),
    "kv4_attention_layout": (ctypes.c_int, [_c_int32, _vp, _c_int64, _vp, _vp, _vp, _vp, _LP, _c_int64, _vp,
                                            _c_int32, _vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32, _c_int32,
                                            _c_int32, _c_int32, _c_int32, _c_int32, _c_uint64, _c_int32,
                                            ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "kv4_dequant_layout": (ctypes.c_int, [_c_int32, _vp, _vp, _LP, _c_int64, _vp, _c_int64, _c_int32, _c_int32,
                                          _c_int32, _c_int32, _c_uint64, _c_int32, _vp, _vp]),
}

_lib = None


class Kv4Error(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/kv4.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv4_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded libkv4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkv4.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def kv4_last_error() -> str:
    return lib().kv4_last_error().decode()


def _check(func: str, rc: int):
    if rc != KV4_OK:
        raise Kv4Error(func, rc, kv4_last_error())


def _b(b: Optional[int]) -> int:
    """b as the C calls take it: 0 lets the library derive the largest power
    of two dividing head_size; any other value is passed on and validated
    there."""
    return 0 if b is None else int(b)


def _torch_stream(stream):
    """The torch stream object of the stream a call is queued on: the current
    stream, a torch.cuda.Stream, or a raw hipStream_t handle."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _empty_on(stream, shape, dtype, device) -> torch.Tensor:
    """A buffer the binding allocates for a call (its output or workspace),
    taken from the caching allocator's pool of the call's own stream: when
    the binding drops it, the allocator hands it out again only for work
    queued after this call on that stream, never while the call's kernels
    may still write it."""
    with torch.cuda.stream(_torch_stream(stream)):
        return torch.empty(shape, dtype=dtype, device=device)


def _need(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kv4_rht_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                  value_cache: torch.Tensor, k_scale_cache: torch.Tensor, v_scale_cache: torch.Tensor,
                  slot_mapping: torch.Tensor, sign_seed: int = DEFAULT_SIGN_SEED,
                  b: Optional[int] = None, stream=None) -> None:
    """Rotate, quantize and scatter key/value [T, nkv, hs] (bf16) into the
    int4 caches [nb, bs, nkv, hs/2] (uint8) and scale caches [nb, bs, nkv]
    (float32) at slot_mapping [T] (int64). Asynchronous on `stream`."""
    _need(key, "key", torch.bfloat16, 3)
    _need(value, "value", torch.bfloat16, 3)
    _need(key_cache, "key_cache", torch.uint8, 4)
    _need(value_cache, "value_cache", torch.uint8, 4)
    _need(k_scale_cache, "k_scale_cache", torch.float32, 3)
    _need(v_scale_cache, "v_scale_cache", torch.float32, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"), (k_scale_cache, "k_scale_cache"),
                 (v_scale_cache, "v_scale_cache"), (slot_mapping, "slot_mapping")):
        _contig(t, n)
    T, nkv, hs = key.shape
    nb, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or slot_mapping.shape[0] != T:
        raise ValueError("key/value/slot_mapping shapes disagree")
    if key_cache.shape != (nb, bs, nkv, hs // 2) or value_cache.shape != key_cache.shape:
        raise ValueError(f"caches must be [num_blocks, block_size, {nkv}, {hs // 2}]")
    if k_scale_cache.shape != (nb, bs, nkv) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError(f"scale caches must be [num_blocks, block_size, {nkv}]")
    for t, n in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != hs:
            raise ValueError(f"{n} must have contiguous heads (stride (*, {hs}, 1))")
    rc = lib().kv4_rht_write(key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0),
                             key_cache.data_ptr(), value_cache.data_ptr(), k_scale_cache.data_ptr(),
                             v_scale_cache.data_ptr(), slot_mapping.data_ptr(), T, nkv, hs,
                             _b(b), bs, nb, sign_seed & (2 ** 64 - 1), _stream(stream))
    _check("kv4_rht_write", rc)


def kv4_paged_attention_workspace_size(num_q_tokens: int, num_seqs: int, num_q_heads: int,
                                       num_kv_heads: int, head_size: int, max_query_len: int,
                                       max_seq_len: int) -> int:
    n = lib().kv4_paged_attention_workspace_size(num_q_tokens, num_seqs, num_q_heads, num_kv_heads,
                                                 head_size, max_query_len, max_seq_len)
    err = kv4_last_error()
    if n == 0 and err:
        raise Kv4Error("kv4_paged_attention_workspace_size", KV4_EINVAL, err)
    return int(n)


def kv4_paged_attention(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                        k_scale_cache: torch.Tensor, v_scale_cache: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                        max_query_len: int, max_seq_len: int, softmax_scale: Optional[float] = None,
                        sign_seed: int = DEFAULT_SIGN_SEED, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, b: Optional[int] = None,
                        stream=None) -> torch.Tensor:
    """Paged causal attention over the int4 RHT cache. query [Tq, nq, hs] bf16,
    block_table [S, max_blocks] int32, seq_lens [S] int32, query_start_loc
    [S+1] int32 (device), max_query_len / max_seq_len host ints. Returns out
    [Tq, nq, hs] bf16. Asynchronous on `stream`."""
    _need(query, "query", torch.bfloat16, 3)
    _need(key_cache, "key_cache", torch.uint8, 4)
    _need(value_cache, "value_cache", torch.uint8, 4)
    _need(k_scale_cache, "k_scale_cache", torch.float32, 3)
    _need(v_scale_cache, "v_scale_cache", torch.float32, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"), (k_scale_cache, "k_scale_cache"),
                 (v_scale_cache, "v_scale_cache"), (block_table, "block_table"), (seq_lens, "seq_lens"),
                 (query_start_loc, "query_start_loc")):
        _contig(t, n)
    Tq, nq, hs = query.shape
    nb, bs, nkv = key_cache.shape[0], key_cache.shape[1], key_cache.shape[2]
    S = seq_lens.shape[0]
    if key_cache.shape[3] != hs // 2 or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with query head_size")
    if k_scale_cache.shape != (nb, bs, nkv) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError("scale cache shapes disagree with the caches")
    if query_start_loc.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("query_start_loc must be [num_seqs + 1] and block_table [num_seqs, *]")
    if query.stride(2) != 1 or query.stride(1) != hs:
        raise ValueError("query must have contiguous heads")
    if out is None:
        out = _empty_on(stream, (Tq, nq, hs), torch.bfloat16, query.device)
    _need(out, "out", torch.bfloat16, 3)
    _contig(out, "out")
    if out.shape != (Tq, nq, hs):
        raise ValueError("out must be [num_q_tokens, num_q_heads, head_size]")
    need = kv4_paged_attention_workspace_size(Tq, S, nq, nkv, hs, max_query_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = _empty_on(stream, (need,), torch.uint8, query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if softmax_scale is None:
        softmax_scale = hs ** -0.5
    rc = lib().kv4_paged_attention(
        query.data_ptr(), query.stride(0), key_cache.data_ptr(), value_cache.data_ptr(),
        k_scale_cache.data_ptr(), v_scale_cache.data_ptr(), nb, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), query_start_loc.data_ptr(), S, Tq,
        int(max_query_len), int(max_seq_len), nq, nkv, hs, _b(b), bs,
        sign_seed & (2 ** 64 - 1), float(softmax_scale), out.data_ptr(), ws_ptr, ws_bytes, _stream(stream))
    _check("kv4_paged_attention", rc)
    return out


KV4_NOALLOC_SCRATCH_BYTES = 64 << 20


def kv4_paged_attention_noalloc(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                                k_scale_cache: torch.Tensor, v_scale_cache: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                                max_query_len: int, max_seq_len: int, out: torch.Tensor,
                                softmax_scale: Optional[float] = None, sign_seed: int = DEFAULT_SIGN_SEED,
                                b: Optional[int] = None, stream=None) -> torch.Tensor:
    """kv4_paged_attention without a workspace and without any allocation:
    the caller passes `out` (bf16 [Tq, nq, hs]); the split partials use the
    library's static per-GPU scratch (KV4_NOALLOC_SCRATCH_BYTES). Calls whose
    kernels may overlap on one GPU race on that scratch."""
    for t, n, dt, nd in ((query, "query", torch.bfloat16, 3), (key_cache, "key_cache", torch.uint8, 4),
                         (value_cache, "value_cache", torch.uint8, 4), (k_scale_cache, "k_scale_cache", torch.float32, 3),
                         (v_scale_cache, "v_scale_cache", torch.float32, 3), (block_table, "block_table", torch.int32, 2),
                         (seq_lens, "seq_lens", torch.int32, 1), (query_start_loc, "query_start_loc", torch.int32, 1),
                         (out, "out", torch.bfloat16, 3)):
        _need(t, n, dt, nd)
        if n != "query":
            _contig(t, n)
    Tq, nq, hs = query.shape
    nb, bs, nkv = key_cache.shape[0], key_cache.shape[1], key_cache.shape[2]
    S = seq_lens.shape[0]
    if key_cache.shape[3] != hs // 2 or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with query head_size")
    if k_scale_cache.shape != (nb, bs, nkv) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError("scale cache shapes disagree with the caches")
    if query_start_loc.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("query_start_loc must be [num_seqs + 1] and block_table [num_seqs, *]")
    if query.stride(2) != 1 or query.stride(1) != hs:
        raise ValueError("query must have contiguous heads")
    if out.shape != (Tq, nq, hs):
        raise ValueError("out must be [num_q_tokens, num_q_heads, head_size]")
    if softmax_scale is None:
        softmax_scale = hs ** -0.5
    rc = lib().kv4_paged_attention_noalloc(
        query.data_ptr(), query.stride(0), key_cache.data_ptr(), value_cache.data_ptr(),
        k_scale_cache.data_ptr(), v_scale_cache.data_ptr(), nb, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), query_start_loc.data_ptr(), S, Tq,
        int(max_query_len), int(max_seq_len), nq, nkv, hs, _b(b), bs,
        sign_seed & (2 ** 64 - 1), float(softmax_scale), out.data_ptr(), _stream(stream))
    _check("kv4_paged_attention_noalloc", rc)
    return out


def kv4_dequant(cache: torch.Tensor, scale_cache: torch.Tensor, slot_mapping: torch.Tensor,
                inverse_rotate: bool = False, sign_seed: int = DEFAULT_SIGN_SEED,
                out: Optional[torch.Tensor] = None, b: Optional[int] = None, stream=None) -> torch.Tensor:
    """Gather slots from an int4 cache and dequantize to float32 [T, nkv, hs];
    with inverse_rotate, map back to the original domain (D.H(.)/b)."""
    _need(cache, "cache", torch.uint8, 4)
    _need(scale_cache, "scale_cache", torch.float32, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    for t, n in ((cache, "cache"), (scale_cache, "scale_cache"), (slot_mapping, "slot_mapping")):
        _contig(t, n)
    nb, bs, nkv, half = cache.shape
    hs = 2 * half
    T = slot_mapping.shape[0]
    if out is None:
        out = _empty_on(stream, (T, nkv, hs), torch.float32, cache.device)
    _need(out, "out", torch.float32, 3)
    _contig(out, "out")
    rc = lib().kv4_dequant(cache.data_ptr(), scale_cache.data_ptr(), nb, slot_mapping.data_ptr(), T, nkv,
                           hs, _b(b), bs, sign_seed & (2 ** 64 - 1),
                           1 if inverse_rotate else 0, out.data_ptr(), _stream(stream))
    _check("kv4_dequant", rc)
    return out


def kv4_stream_read(buffer: torch.Tensor, sink: torch.Tensor, grid: int = 2048, stream=None) -> None:
    """Read every byte of `buffer` once (bandwidth calibration; see
    include/kv4.h). `sink` is a 4-byte device tensor."""
    _contig(buffer, "buffer")
    if buffer.device.type != "cuda" or sink.device.type != "cuda" or sink.numel() * sink.element_size() < 4:
        raise ValueError("buffer and a 4-byte sink must be GPU tensors")
    nbytes = buffer.numel() * buffer.element_size()
    _check("kv4_stream_read", lib().kv4_stream_read(buffer.data_ptr(), nbytes - nbytes % 16, sink.data_ptr(),
                                                    int(grid), _stream(stream)))


KV4_DEBUG_SLOT, KV4_DEBUG_PAGE, KV4_DEBUG_SEQLEN, KV4_DEBUG_QSL = 1, 2, 4, 8


def kv4_debug_flags(clear: bool = False) -> int:
    """KV4_DEBUG_* bits of the inputs the kernels clamped or skipped (a
    library built with -DKV4_DEBUG, selected with KV4_LIBRARY; see
    include/kv4.h). Synchronizes the device."""
    v = ctypes.c_uint32(0)
    _check("kv4_debug_flags", lib().kv4_debug_flags(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


__all__ = ["kv4_rht_write", "kv4_paged_attention", "kv4_paged_attention_workspace_size", "kv4_dequant",
           "kv4_last_error", "Kv4Error", "lib", "header_functions", "LIB_PATH"]


def _mode(kv_quant_mode) -> int:
    if kv_quant_mode not in _MODES:
        raise ValueError(f"kv_quant_mode must be 'int8' or 'fp8', got {kv_quant_mode!r}")
    return _MODES[kv_quant_mode]


def kv4_pth_write(kv_quant_mode, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                  value_cache: torch.Tensor, k_scale_cache: torch.Tensor, v_scale_cache: torch.Tensor,
                  slot_mapping: torch.Tensor, stream=None) -> None:
    """Quantize key/value [T, nkv, hs] (bf16) per (token, kv head) to int8 or
    fp8 e4m3fn codes ('int8' / 'fp8'; no rotation) into the caches
    [nb, bs, nkv, hs] (uint8) and scale caches [nb, bs, nkv] (float32) at
    slot_mapping [T] (int64). Asynchronous on `stream`."""
    m = _mode(kv_quant_mode)
    _need(key, "key", torch.bfloat16, 3)
    _need(value, "value", torch.bfloat16, 3)
    _need(key_cache, "key_cache", torch.uint8, 4)
    _need(value_cache, "value_cache", torch.uint8, 4)
    _need(k_scale_cache, "k_scale_cache", torch.float32, 3)
    _need(v_scale_cache, "v_scale_cache", torch.float32, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"), (k_scale_cache, "k_scale_cache"),
                 (v_scale_cache, "v_scale_cache"), (slot_mapping, "slot_mapping")):
        _contig(t, n)
    T, nkv, hs = key.shape
    nb, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or slot_mapping.shape[0] != T:
        raise ValueError("key/value/slot_mapping shapes disagree")
    if key_cache.shape != (nb, bs, nkv, hs) or value_cache.shape != key_cache.shape:
        raise ValueError(f"caches must be [num_blocks, block_size, {nkv}, {hs}]")
    if k_scale_cache.shape != (nb, bs, nkv) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError(f"scale caches must be [num_blocks, block_size, {nkv}]")
    for t, n in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != hs:
            raise ValueError(f"{n} must have contiguous heads (stride (*, {hs}, 1))")
    rc = lib().kv4_pth_write(m, key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0),
                             key_cache.data_ptr(), value_cache.data_ptr(), k_scale_cache.data_ptr(),
                             v_scale_cache.data_ptr(), slot_mapping.data_ptr(), T, nkv, hs, bs, nb, _stream(stream))
    _check("kv4_pth_write", rc)


def kv4_pth_dequant(kv_quant_mode, cache: torch.Tensor, scale_cache: torch.Tensor, slot_mapping: torch.Tensor,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gather slots from an int8 / fp8 cache and dequantize to float32 [T, nkv, hs]."""
    m = _mode(kv_quant_mode)
    _need(cache, "cache", torch.uint8, 4)
    _need(scale_cache, "scale_cache", torch.float32, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    for t, n in ((cache, "cache"), (scale_cache, "scale_cache"), (slot_mapping, "slot_mapping")):
        _contig(t, n)
    nb, bs, nkv, hs = cache.shape
    if scale_cache.shape != (nb, bs, nkv):
        raise ValueError("scale cache shape disagrees with the cache")
    T = slot_mapping.shape[0]
    if out is None:
        out = _empty_on(stream, (T, nkv, hs), torch.float32, cache.device)
    _need(out, "out", torch.float32, 3)
    _contig(out, "out")
    if out.shape != (T, nkv, hs):
        raise ValueError("out must be [num_tokens, num_kv_heads, head_size]")
    rc = lib().kv4_pth_dequant(m, cache.data_ptr(), scale_cache.data_ptr(), nb, slot_mapping.data_ptr(), T, nkv,
                               hs, bs, out.data_ptr(), _stream(stream))
    _check("kv4_pth_dequant", rc)
    return out


def kv4_pth_attention_workspace_size(kv_quant_mode, num_q_tokens: int, num_seqs: int, num_q_heads: int,
                                     num_kv_heads: int, head_size: int, max_query_len: int,
                                     max_seq_len: int) -> int:
    n = lib().kv4_pth_attention_workspace_size(_mode(kv_quant_mode), num_q_tokens, num_seqs, num_q_heads,
                                               num_kv_heads, head_size, max_query_len, max_seq_len)
    err = kv4_last_error()
    if n == 0 and err:
        raise Kv4Error("kv4_pth_attention_workspace_size", KV4_EINVAL, err)
    return int(n)


def kv4_pth_attention(kv_quant_mode, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      k_scale_cache: torch.Tensor, v_scale_cache: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, query_start_loc: torch.Tensor, max_query_len: int,
                      max_seq_len: int, softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Paged causal attention over an int8 / fp8 per-token-head cache
    [nb, bs, nkv, hs] (no rotation); other arguments as kv4_paged_attention."""
    m = _mode(kv_quant_mode)
    _need(query, "query", torch.bfloat16, 3)
    _need(key_cache, "key_cache", torch.uint8, 4)
    _need(value_cache, "value_cache", torch.uint8, 4)
    _need(k_scale_cache, "k_scale_cache", torch.float32, 3)
    _need(v_scale_cache, "v_scale_cache", torch.float32, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"), (k_scale_cache, "k_scale_cache"),
                 (v_scale_cache, "v_scale_cache"), (block_table, "block_table"), (seq_lens, "seq_lens"),
                 (query_start_loc, "query_start_loc")):
        _contig(t, n)
    Tq, nq, hs = query.shape
    nb, bs, nkv = key_cache.shape[0], key_cache.shape[1], key_cache.shape[2]
    S = seq_lens.shape[0]
    if key_cache.shape[3] != hs or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with query head_size")
    if k_scale_cache.shape != (nb, bs, nkv) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError("scale cache shapes disagree with the caches")
    if query_start_loc.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("query_start_loc must be [num_seqs + 1] and block_table [num_seqs, *]")
    if query.stride(2) != 1 or query.stride(1) != hs:
        raise ValueError("query must have contiguous heads")
    if out is None:
        out = _empty_on(stream, (Tq, nq, hs), torch.bfloat16, query.device)
    _need(out, "out", torch.bfloat16, 3)
    _contig(out, "out")
    if out.shape != (Tq, nq, hs):
        raise ValueError("out must be [num_q_tokens, num_q_heads, head_size]")
    need = kv4_pth_attention_workspace_size(m, Tq, S, nq, nkv, hs, max_query_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = _empty_on(stream, (need,), torch.uint8, query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if softmax_scale is None:
        softmax_scale = hs ** -0.5
    rc = lib().kv4_pth_attention(
        m, query.data_ptr(), query.stride(0), key_cache.data_ptr(), value_cache.data_ptr(),
        k_scale_cache.data_ptr(), v_scale_cache.data_ptr(), nb, block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), query_start_loc.data_ptr(), S, Tq, int(max_query_len), int(max_seq_len), nq, nkv,
        hs, bs, float(softmax_scale), out.data_ptr(), ws_ptr, ws_bytes, _stream(stream))
    _check("kv4_pth_attention", rc)
    return out


# ---------------------------------------------------------------------------
# Caller-described cache layouts (all three modes; see include/kv4.h)
# ---------------------------------------------------------------------------
_ANY_MODES = {"int4": 0, 0: 0, "int8": KV4_MODE_INT8, "fp8": KV4_MODE_FP8, KV4_MODE_INT8: KV4_MODE_INT8,
              KV4_MODE_FP8: KV4_MODE_FP8}


def _any_mode(m) -> int:
    if m not in _ANY_MODES:
        raise ValueError(f"kv_quant_mode must be 'int4', 'int8' or 'fp8', got {m!r}")
    return _ANY_MODES[m]


def kv4_cache_layout_packed(kv_quant_mode, num_kv_heads: int, head_size: int, block_size: int) -> CacheLayout:
    lay = CacheLayout()
    _check("kv4_cache_layout_packed",
           lib().kv4_cache_layout_packed(_any_mode(kv_quant_mode), num_kv_heads, head_size, block_size,
                                         ctypes.byref(lay)))
    return lay


def kv4_cache_layout_inline(kv_quant_mode, num_kv_heads: int, head_size: int, block_size: int):
    """(layout, block_bytes, value_offset, scale_offset) of the inline-scale
    padded-slot layout."""
    lay = CacheLayout()
    bb, vo, so = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("kv4_cache_layout_inline",
           lib().kv4_cache_layout_inline(_any_mode(kv_quant_mode), num_kv_heads, head_size, block_size,
                                         ctypes.byref(lay), ctypes.byref(bb), ctypes.byref(vo), ctypes.byref(so)))
    return lay, bb.value, vo.value, so.value


class LayoutCache:
    """A K/V cache pair with its scales in a caller-described layout: device
    pointers of the K codes, V codes, K scales and V scales, the layout, and
    the tensor(s) that own the memory."""

    def __init__(self, mode, layout: CacheLayout, num_blocks: int, block_size: int, num_kv_heads: int,
                 head_size: int, key_ptr: int, value_ptr: int, k_scale_ptr: int, v_scale_ptr: int, owners=()):
        self.mode = _any_mode(mode)
        self.layout = layout
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_size = num_kv_heads, head_size
        self.key_ptr, self.value_ptr, self.k_scale_ptr, self.v_scale_ptr = key_ptr, value_ptr, k_scale_ptr, v_scale_ptr
        self.owners = tuple(owners)

    @classmethod
    def inline(cls, mode, num_blocks: int, block_size: int, num_kv_heads: int, head_size: int,
               device="cuda", fill: int = 0):
        """One uint8 buffer [num_blocks, block_bytes] in the inline-scale layout."""
        lay, bb, vo, so = kv4_cache_layout_inline(mode, num_kv_heads, head_size, block_size)
        buf = torch.full((num_blocks, bb), fill, dtype=torch.uint8, device=device)
        p = buf.data_ptr()
        c = cls(mode, lay, num_blocks, block_size, num_kv_heads, head_size, p, p + vo, p + so, p + vo + so, (buf,))
        c.buffer, c.block_bytes, c.value_offset, c.scale_offset = buf, bb, vo, so
        return c


def kv4_write_layout(key: torch.Tensor, value: torch.Tensor, cache: LayoutCache, slot_mapping: torch.Tensor,
                     sign_seed: int = DEFAULT_SIGN_SEED, b: Optional[int] = None, stream=None) -> None:
    """Write path of the cache's mode into a LayoutCache (see kv4_rht_write /
    kv4_pth_write)."""
    _need(key, "key", torch.bfloat16, 3)
    _need(value, "value", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    _contig(slot_mapping, "slot_mapping")
    T, nkv, hs = key.shape
    if value.shape != key.shape or slot_mapping.shape[0] != T:
        raise ValueError("key/value/slot_mapping shapes disagree")
    if (nkv, hs) != (cache.num_kv_heads, cache.head_size):
        raise ValueError("key heads / head size disagree with the cache")
    for t, n in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != hs:
            raise ValueError(f"{n} must have contiguous heads (stride (*, {hs}, 1))")
    rc = lib().kv4_write_layout(cache.mode, key.data_ptr(), value.data_ptr(), key.stride(0), value.stride(0),
                                cache.key_ptr, cache.value_ptr, cache.k_scale_ptr, cache.v_scale_ptr,
                                ctypes.byref(cache.layout), slot_mapping.data_ptr(), T, nkv, hs,
                                _b(b), cache.block_size, cache.num_blocks,
                                sign_seed & (2 ** 64 - 1), _stream(stream))
    _check("kv4_write_layout", rc)


def kv4_attention_layout_workspace_size(cache: LayoutCache, num_q_tokens: int, num_seqs: int, num_q_heads: int,
                                        max_query_len: int, max_seq_len: int) -> int:
    n = lib().kv4_attention_layout_workspace_size(cache.mode, ctypes.byref(cache.layout), num_q_tokens, num_seqs,
                                                  num_q_heads, cache.num_kv_heads, cache.head_size, max_query_len,
                                                  max_seq_len)
    err = kv4_last_error()
    if n == 0 and err:
        raise Kv4Error("kv4_attention_layout_workspace_size", KV4_EINVAL, err)
    return int(n)


def kv4_attention_layout(query: torch.Tensor, cache: LayoutCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                         query_start_loc: torch.Tensor, max_query_len: int, max_seq_len: int,
                         sign_seed: int = DEFAULT_SIGN_SEED, softmax_scale: Optional[float] = None,
                         b: Optional[int] = None, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         sliding_window: int = 0) -> torch.Tensor:
    """Paged causal attention over a LayoutCache (see kv4_paged_attention /
    kv4_pth_attention); sliding_window > 0 keeps the window most recent keys
    of each query's causal range."""
    _need(query, "query", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc")):
        _contig(t, n)
    Tq, nq, hs = query.shape
    S = seq_lens.shape[0]
    if hs != cache.head_size:
        raise ValueError("query head size disagrees with the cache")
    if query_start_loc.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("query_start_loc must be [num_seqs + 1] and block_table [num_seqs, *]")
    if query.stride(2) != 1 or query.stride(1) != hs:
        raise ValueError("query must have contiguous heads")
    if out is None:
        out = _empty_on(stream, (Tq, nq, hs), torch.bfloat16, query.device)
    _need(out, "out", torch.bfloat16, 3)
    _contig(out, "out")
    need = kv4_attention_layout_workspace_size(cache, Tq, S, nq, max_query_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = _empty_on(stream, (need,), torch.uint8, query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if softmax_scale is None:
        softmax_scale = hs ** -0.5
    rc = lib().kv4_attention_layout(
        cache.mode, query.data_ptr(), query.stride(0), cache.key_ptr, cache.value_ptr, cache.k_scale_ptr,
        cache.v_scale_ptr, ctypes.byref(cache.layout), cache.num_blocks, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), query_start_loc.data_ptr(), S, Tq, int(max_query_len),
        int(max_seq_len), nq, cache.num_kv_heads, hs, _b(b), cache.block_size,
        sign_seed & (2 ** 64 - 1), int(sliding_window), float(softmax_scale), out.data_ptr(), ws_ptr, ws_bytes,
        _stream(stream))
    _check("kv4_attention_layout", rc)
    return out


def kv4_dequant_layout(cache: LayoutCache, which: str, slot_mapping: torch.Tensor, inverse_rotate: bool = False,
                       sign_seed: int = DEFAULT_SIGN_SEED, b: Optional[int] = None, stream=None) -> torch.Tensor:
    """Gather and dequantize K ('k') or V ('v') slots of a LayoutCache
    (float32 [T, nkv, hs]; out-of-range slots give zeros)."""
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    _contig(slot_mapping, "slot_mapping")
    if which not in ("k", "v"):
        raise ValueError("which must be 'k' or 'v'")
    T = slot_mapping.shape[0]
    hs, nkv = cache.head_size, cache.num_kv_heads
    out = _empty_on(stream, (T, nkv, hs), torch.float32, slot_mapping.device)
    codes, scales = (cache.key_ptr, cache.k_scale_ptr) if which == "k" else (cache.value_ptr, cache.v_scale_ptr)
    rc = lib().kv4_dequant_layout(cache.mode, codes, scales, ctypes.byref(cache.layout), cache.num_blocks,
                                  slot_mapping.data_ptr(), T, nkv, hs, _b(b),
                                  cache.block_size, sign_seed & (2 ** 64 - 1), 1 if inverse_rotate else 0,
                                  out.data_ptr(), _stream(stream))
    _check("kv4_dequant_layout", rc)
    return out


def packed_layout_cache(mode, key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale_cache: torch.Tensor,
                        v_scale_cache: torch.Tensor) -> LayoutCache:
    """A LayoutCache view of packed caches ([nb, bs, nkv, C] codes, [nb, bs,
    nkv] scales), for the *_layout entry points."""
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"), (k_scale_cache, "k_scale_cache"),
                 (v_scale_cache, "v_scale_cache")):
        _contig(t, n)
    m = _any_mode(mode)
    nb, bs, nkv, c = key_cache.shape
    hs = 2 * c if m == 0 else c
    lay = kv4_cache_layout_packed(m, nkv, hs, bs)
    return LayoutCache(m, lay, nb, bs, nkv, hs, key_cache.data_ptr(), value_cache.data_ptr(),
                       k_scale_cache.data_ptr(), v_scale_cache.data_ptr(),
                       (key_cache, value_cache, k_scale_cache, v_scale_cache))
