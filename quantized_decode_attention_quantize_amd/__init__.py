"""kvq: K4V2 group-128 quantised paged KV cache for AMD Instinct MI355X.

A thin ctypes binding over ``libkvq.so`` (hand-written HIP kernels for gfx950,
C ABI declared in ``include/kvq.h``).  The binding only marshals arguments:
every step of quantise-append and decode attention runs in the library's
kernels.  PyTorch provides device memory and streams.  There is no CPU
fallback: if the library is missing, every call raises.

Names follow the C ABI: ``quantize_append`` and ``decode_attention``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "KvqError", "Format", "load", "library_path", "format_from_string", "page_bytes",
    "cache_bytes", "alloc_cache", "quantize_append", "decode_workspace_bytes",
    "decode_pages_per_split", "alloc_workspace", "decode_attention", "decode_partials",
    "decode_combine", "append_decode_attention", "append_decode_partials", "append_decode_attention_noalloc",
    "NOALLOC_SCRATCH_BYTES", "decode_split_slots",
    "decode_partials_slots", "decode_combine_slots", "version",
    "HEAD_DIM", "PAGE", "REGION_BYTES", "KEY_NORM_GROUP", "KEY_NORM_PAGE",
]

HEAD_DIM = 128
PAGE = 16
NOALLOC_SCRATCH_BYTES = 16 << 20     # KVQ_NOALLOC_SCRATCH_BYTES of include/kvq.h
REGION_BYTES = 1664

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq.so")
_lib = None

KVQ_OK = 0
_STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_NULL", 2: "KVQ_ERR_SHAPE", 3: "KVQ_ERR_UNSUPPORTED",
           4: "KVQ_ERR_ALIGN", 5: "KVQ_ERR_WORKSPACE", 6: "KVQ_ERR_HIP"}
OUT_F16, OUT_F32 = 0, 1


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {_STATUS.get(status, status)}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


KEY_NORM_GROUP = 0      # each token's key group normalised on its own (v1)
KEY_NORM_PAGE = 1       # page-balanced keys: per-page column scales


class Format(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("key_norm", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkvq.so (built in-tree by ``build.py``).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libkvq.so not found at {_LIB_PATH}; build it with "
                           "`python -m quantized_decode_attention_quantize_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    FP = ctypes.POINTER(Format)
    sigs = {
        "kvq_format_from_string": (ctypes.c_int, [ctypes.c_char_p, FP]),
        "kvq_page_bytes": (sz, [FP]),
        "kvq_cache_bytes": (sz, [FP, i64, i32]),
        "kvq_quantize_append": (ctypes.c_int, [FP, P, P, i64, i64, P, i64, i32, P, i64, P]),
        "kvq_decode_workspace_bytes": (sz, [FP, i32, i32, i32, i32, i32]),
        "kvq_decode_pages_per_split": (i32, [i32, i32, i32, i32]),
        "kvq_decode_attention": (ctypes.c_int, [FP, P, ctypes.c_int, P, P, i64, P, i32, P, i32, i32,
                                                i32, i32, ctypes.c_float, P, sz, P]),
        "kvq_decode_attention_ex": (ctypes.c_int, [FP, P, ctypes.c_int, P, P, i64, P, i32, P, i32,
                                                   i32, i32, i32, ctypes.c_float, P, sz, i32, P]),
        "kvq_decode_partials": (ctypes.c_int, [FP, P, P, i64, P, i32, P, i32, i32, i32, i32,
                                               ctypes.c_float, P, sz, i32, P]),
        "kvq_decode_combine": (ctypes.c_int, [FP, P, ctypes.c_int, P, i32, i32, i32, i32, P, sz, i32, P]),
        "kvq_append_decode_attention": (ctypes.c_int, [FP, P, ctypes.c_int, P, P, i64, i64, P, P, i64, P, i32,
                                                       P, i32, i32, i32, i32, ctypes.c_float, P, sz, i32, P]),
        "kvq_append_decode_partials": (ctypes.c_int, [FP, P, P, i64, i64, P, P, i64, P, i32, P, i32, i32, i32,
                                                      i32, ctypes.c_float, P, sz, i32, P]),
        "kvq_append_decode_attention_noalloc": (ctypes.c_int, [FP, P, ctypes.c_int, P, P, i64, i64, P, P, i64, P,
                                                               i32, P, i32, i32, i32, i32, ctypes.c_float, i32, P]),
        "kvq_decode_workspace_bytes_mq": (sz, [FP, i32, i32, i32, i32, i32, i32]),
        "kvq_decode_attention_mq": (ctypes.c_int, [FP, P, ctypes.c_int, P, i32, P, i64, P, i32, P, i32, i32,
                                                   i32, i32, ctypes.c_float, P, sz, i32, P]),
        "kvq_set_split_kernel_events": (ctypes.c_int, [P, P]),
        "kvq_stream_read_probe": (ctypes.c_int, [P, sz, P, P]),
        "kvq_page_walk_probe": (ctypes.c_int, [FP, P, i64, P, i32, P, i32, i32, i32, i32, P, P]),
        "kvq_decode_split_slots": (i32, [FP, i32, i32, i32, i32, i32]),
        "kvq_decode_partials_slots": (ctypes.c_int, [FP, P, P, i64, P, i32, P, i32, i32, i32, i32,
                                                     ctypes.c_float, P, sz, i32, i32, i32, i32, P]),
        "kvq_decode_combine_slots": (ctypes.c_int, [P, ctypes.c_int, i32, i32, P, sz, i32, i32, P]),
        "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kvq_last_hip_error": (ctypes.c_int, []),
        "kvq_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != KVQ_OK:
        lib = load()
        raise KvqError(status, what, lib.kvq_last_hip_error() if status == 6 else 0)


def version() -> str:
    return load().kvq_version().decode()


def format_from_string(preset: str = "kvarn_k4v2_g128", page_tokens: int = 16) -> Format:
    """The preset's format; page_tokens (16, 32, 64, 128 for the quantised
    presets) sets tokens per page (block_size)."""
    f = Format()
    _check(load().kvq_format_from_string(preset.encode(), ctypes.byref(f)), "format_from_string")
    f.block_size = page_tokens
    if page_bytes(f) == 0:
        raise KvqError(3, f"page size {page_tokens} not supported for {preset}")
    return f


_V1 = None


def _fmt(fmt: Format | None) -> Format:
    global _V1
    if fmt is not None:
        return fmt
    if _V1 is None:
        _V1 = format_from_string("k4v2_g128")
    return _V1


def page_bytes(fmt: Format | None = None) -> int:
    return int(load().kvq_page_bytes(ctypes.byref(_fmt(fmt))))


def cache_bytes(num_pages: int, num_kv_heads: int, fmt: Format | None = None) -> int:
    return int(load().kvq_cache_bytes(ctypes.byref(_fmt(fmt)), num_pages, num_kv_heads))


def alloc_cache(num_pages: int, num_kv_heads: int, device="cuda", fmt: Format | None = None) -> torch.Tensor:
    """Uninitialised pool u8 [num_pages][num_kv_heads][page_bytes(fmt)]
    (256 (k_bits + v_bits) + 128 bytes for a quantised preset: 1664 for K4V2;
    8192 for the fp16 baseline)."""
    return torch.empty((num_pages, num_kv_heads, page_bytes(fmt)), dtype=torch.uint8, device=device)


def _region(fmt: Format | None) -> int:
    n = page_bytes(fmt)
    if n == 0:
        raise KvqError(3, "unsupported format")
    return n


def _stream_ptr(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    """Device address of a tensor that lives on the current GPU (the kernels
    dereference it on the device, so a host tensor is refused here)."""
    if not t.is_cuda:
        raise ValueError("kvq operates on GPU tensors; got a tensor on " + str(t.device))
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(t.data_ptr())


def quantize_append(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                    cache: torch.Tensor, stream=None, fmt: Format | None = None) -> None:
    """Quantise fp16 key/value [T][num_kv_heads][128] into the pool at the given
    slots (int64 [T]; page*16 + offset; negative = skip).  With page-balanced
    keys (fmt.key_norm == KEY_NORM_PAGE) tokens 16b .. 16b + 15 form one
    whole-page block, written together (see kvq_quantize_append)."""
    if key.dtype != torch.float16 or value.dtype != torch.float16:
        raise TypeError("key/value must be float16")
    if slot_mapping.dtype != torch.int64 or cache.dtype != torch.uint8:
        raise TypeError("slot_mapping must be int64 and cache uint8")
    if key.dim() != 3 or key.shape != value.shape or key.shape[2] != HEAD_DIM:
        raise ValueError("key/value must be [T][num_kv_heads][128] with equal shapes")
    T, H, _ = key.shape
    for t in (key, value):
        if t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
            raise ValueError("key/value heads must be contiguous 128-element rows")
    if cache.dim() != 3 or cache.shape[1] != H or cache.shape[2] != _region(fmt) or not cache.is_contiguous():
        raise ValueError("cache must be contiguous [num_pages][num_kv_heads][page_bytes]")
    if not slot_mapping.is_contiguous() or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be a contiguous int64 vector of length T")
    st = load().kvq_quantize_append(ctypes.byref(_fmt(fmt)), _ptr(key), _ptr(value), key.stride(0),
                                    value.stride(0), _ptr(slot_mapping), T, H, _ptr(cache),
                                    cache.shape[0], _stream_ptr(stream))
    _check(st, "kvq_quantize_append")


def decode_pages_per_split(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(load().kvq_decode_pages_per_split(num_seqs, num_q_heads, num_kv_heads, max_seq_len))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                           pages_per_split: int = 0, fmt: Format | None = None) -> int:
    n = load().kvq_decode_workspace_bytes(ctypes.byref(_fmt(fmt)), num_seqs, num_q_heads,
                                          num_kv_heads, max_seq_len, pages_per_split)
    if n == 0:
        raise KvqError(2, "kvq_decode_workspace_bytes")
    return int(n)


def alloc_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                    pages_per_split: int = 0, device="cuda", fmt: Format | None = None) -> torch.Tensor:
    """Workspace for split partials (contents need no initialisation)."""
    n = decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, max_seq_len, pages_per_split, fmt)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _decode_checks(query, cache, block_tables, seq_lens, fmt=None):
    if query.dtype != torch.float16 or query.dim() != 3 or query.shape[2] != HEAD_DIM:
        raise ValueError("query must be float16 [B][Hq][128]")
    if not query.is_contiguous():
        raise ValueError("query must be contiguous")
    B = query.shape[0]
    if cache.dim() != 3 or cache.shape[2] != _region(fmt) or not cache.is_contiguous():
        raise ValueError("cache must be contiguous [num_pages][num_kv_heads][page_bytes]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B][max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [B]")


def decode_attention(query: torch.Tensor, cache: torch.Tensor, block_tables: torch.Tensor,
                     seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float | None = None,
                     out: torch.Tensor | None = None, out_dtype=torch.float32,
                     workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                     stream=None, fmt: Format | None = None) -> torch.Tensor:
    """One decode step: query fp16 [B][Hq][128] against the pool; returns
    out [B][Hq][128] (fp32 or fp16)."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    Hkv = cache.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=query.device)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][Hq][128]")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, max_seq_len, pages_per_split, device=query.device, fmt=fmt)
    st = load().kvq_decode_attention_ex(
        ctypes.byref(_fmt(fmt)), _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
        _ptr(query), _ptr(cache), cache.shape[0], _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, Hq, Hkv, int(max_seq_len), float(softmax_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_decode_attention")
    return out


def decode_workspace_bytes_mq(num_seqs: int, q_len: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                              pages_per_split: int = 0, fmt: Format | None = None) -> int:
    n = load().kvq_decode_workspace_bytes_mq(ctypes.byref(_fmt(fmt)), num_seqs, q_len, num_q_heads,
                                             num_kv_heads, max_seq_len, pages_per_split)
    if n == 0:
        raise KvqError(2, "kvq_decode_workspace_bytes_mq")
    return int(n)


def decode_attention_mq(query: torch.Tensor, cache: torch.Tensor, block_tables: torch.Tensor,
                        seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float | None = None,
                        out: torch.Tensor | None = None, out_dtype=torch.float32,
                        workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                        stream=None, fmt: Format | None = None) -> torch.Tensor:
    """Several causal query rows per sequence: query fp16 [B][M][Hq][128]
    (the sequence's last M positions); returns out [B][M][Hq][128]."""
    if query.dtype != torch.float16 or query.dim() != 4 or query.shape[3] != HEAD_DIM or not query.is_contiguous():
        raise ValueError("query must be contiguous float16 [B][M][Hq][128]")
    B, M, Hq, _ = query.shape
    _decode_checks(query.view(B, M * Hq, HEAD_DIM), cache, block_tables, seq_lens, fmt)
    Hkv = cache.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, M, Hq, HEAD_DIM), dtype=out_dtype, device=query.device)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or \
            tuple(out.shape) != (B, M, Hq, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][M][Hq][128]")
    if workspace is None:
        n = decode_workspace_bytes_mq(B, M, Hq, Hkv, max_seq_len, pages_per_split, fmt)
        workspace = torch.empty(n, dtype=torch.uint8, device=query.device)
    st = load().kvq_decode_attention_mq(
        ctypes.byref(_fmt(fmt)), _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
        _ptr(query), M, _ptr(cache), cache.shape[0], _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, Hq, Hkv, int(max_seq_len), float(softmax_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_decode_attention_mq")
    return out


def decode_partials(query: torch.Tensor, cache: torch.Tensor, block_tables: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, workspace: torch.Tensor,
                    softmax_scale: float | None = None, pages_per_split: int = 0,
                    stream=None, fmt: Format | None = None) -> torch.Tensor:
    """Split phase of a decode step: fills `workspace` with the fp32 split
    partials [B][Hq][splits][132] (see include/kvq.h) and returns it."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load().kvq_decode_partials(
        ctypes.byref(_fmt(fmt)), _ptr(query), _ptr(cache), cache.shape[0], _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), B, Hq, cache.shape[1], int(max_seq_len),
        float(softmax_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_decode_partials")
    return workspace


def decode_combine(workspace: torch.Tensor, seq_lens: torch.Tensor, num_q_heads: int, num_kv_heads: int,
                   max_seq_len: int, out: torch.Tensor | None = None, out_dtype=torch.float32,
                   pages_per_split: int = 0, stream=None, fmt: Format | None = None) -> torch.Tensor:
    """Combine phase: merges the partials written by ``decode_partials`` and
    returns out [B][Hq][128] (fp32 or fp16)."""
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [B]")
    B = seq_lens.numel()
    if out is None:
        out = torch.empty((B, num_q_heads, HEAD_DIM), dtype=out_dtype, device=seq_lens.device)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or \
            out.shape != (B, num_q_heads, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][Hq][128]")
    st = load().kvq_decode_combine(
        ctypes.byref(_fmt(fmt)), _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
        _ptr(seq_lens), B, num_q_heads, num_kv_heads, int(max_seq_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_decode_combine")
    return out


def _new_token_checks(new_key, new_value, B, Hkv):
    for t in (new_key, new_value):
        if t.dtype != torch.float16 or t.dim() != 3 or tuple(t.shape) != (B, Hkv, HEAD_DIM):
            raise ValueError("new_key/new_value must be float16 [B][num_kv_heads][128]")
        if t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
            raise ValueError("new_key/new_value heads must be contiguous 128-element rows")


def append_decode_attention(new_key: torch.Tensor, new_value: torch.Tensor, query: torch.Tensor,
                            cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                            max_seq_len: int, softmax_scale: float | None = None, out: torch.Tensor | None = None,
                            out_dtype=torch.float32, workspace: torch.Tensor | None = None,
                            pages_per_split: int = 0, stream=None, fmt: Format | None = None) -> torch.Tensor:
    """One decode step that first appends the new token of every sequence:
    new_key/new_value fp16 [B][num_kv_heads][128] go into token seq_lens[b]-1,
    then attention over seq_lens[b] tokens.  Returns out [B][Hq][128]."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    Hkv = cache.shape[1]
    _new_token_checks(new_key, new_value, B, Hkv)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=query.device)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][Hq][128]")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, max_seq_len, pages_per_split, device=query.device, fmt=fmt)
    st = load().kvq_append_decode_attention(
        ctypes.byref(_fmt(fmt)), _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
        _ptr(new_key), _ptr(new_value), new_key.stride(0), new_value.stride(0), _ptr(query), _ptr(cache),
        cache.shape[0], _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, Hq, Hkv,
        int(max_seq_len), float(softmax_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_append_decode_attention")
    return out


def append_decode_attention_noalloc(new_key: torch.Tensor, new_value: torch.Tensor, query: torch.Tensor,
                                    cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                    max_seq_len: int, out: torch.Tensor, softmax_scale: float | None = None,
                                    pages_per_split: int = 0, stream=None, fmt: Format | None = None) -> torch.Tensor:
    """``append_decode_attention`` with its split partials in the library's
    fixed device array (kvq_append_decode_attention_noalloc): no workspace,
    and nothing allocated -- ``out`` (fp32 or fp16 [B][Hq][128]) is
    required.  Calls that overlap on one device race on the array."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    Hkv = cache.shape[1]
    _new_token_checks(new_key, new_value, B, Hkv)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][Hq][128]")
    st = load().kvq_append_decode_attention_noalloc(
        ctypes.byref(_fmt(fmt)), _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
        _ptr(new_key), _ptr(new_value), new_key.stride(0), new_value.stride(0), _ptr(query), _ptr(cache),
        cache.shape[0], _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, Hq, Hkv,
        int(max_seq_len), float(softmax_scale), int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_append_decode_attention_noalloc")
    return out


def append_decode_partials(new_key: torch.Tensor, new_value: torch.Tensor, query: torch.Tensor,
                           cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, workspace: torch.Tensor, softmax_scale: float | None = None,
                           pages_per_split: int = 0, stream=None, fmt: Format | None = None) -> torch.Tensor:
    """Split phase of ``append_decode_attention``; ``decode_combine`` finishes it."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    Hkv = cache.shape[1]
    _new_token_checks(new_key, new_value, B, Hkv)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load().kvq_append_decode_partials(
        ctypes.byref(_fmt(fmt)), _ptr(new_key), _ptr(new_value), new_key.stride(0), new_value.stride(0),
        _ptr(query), _ptr(cache), cache.shape[0], _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
        B, Hq, Hkv, int(max_seq_len), float(softmax_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(pages_per_split), _stream_ptr(stream))
    _check(st, "kvq_append_decode_partials")
    return workspace


def decode_split_slots(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                       pages_per_split: int = 0, fmt: Format | None = None) -> int:
    """Partial slots a partials call over one cache with these sizes uses."""
    n = load().kvq_decode_split_slots(ctypes.byref(_fmt(fmt)), num_seqs, num_q_heads, num_kv_heads,
                                      max_seq_len, pages_per_split)
    if n <= 0:
        raise KvqError(2, "kvq_decode_split_slots")
    return int(n)


def decode_partials_slots(query: torch.Tensor, cache: torch.Tensor, block_tables: torch.Tensor,
                          seq_lens: torch.Tensor, max_seq_len: int, workspace: torch.Tensor, slot_offset: int,
                          total_slots: int, rotated: bool = True, softmax_scale: float | None = None,
                          pages_per_split: int = 0, stream=None, fmt: Format | None = None) -> torch.Tensor:
    """Partials of one cache into slots [slot_offset, slot_offset + splits) of a
    workspace of fp32 [B][Hq][total_slots][132] (see include/kvq.h)."""
    _decode_checks(query, cache, block_tables, seq_lens, fmt)
    B, Hq, _ = query.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    st = load().kvq_decode_partials_slots(
        ctypes.byref(_fmt(fmt)), _ptr(query), _ptr(cache), cache.shape[0], _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), B, Hq, cache.shape[1], int(max_seq_len), float(softmax_scale),
        _ptr(workspace), workspace.numel() * workspace.element_size(), int(pages_per_split), int(slot_offset),
        int(total_slots), int(bool(rotated)), _stream_ptr(stream))
    _check(st, "kvq_decode_partials_slots")
    return workspace


def decode_combine_slots(workspace: torch.Tensor, num_seqs: int, num_q_heads: int, total_slots: int,
                         rotated: bool = True, out: torch.Tensor | None = None, out_dtype=torch.float32,
                         stream=None) -> torch.Tensor:
    """Merge all slots of every row of a slotted workspace into out [B][Hq][128]."""
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, HEAD_DIM), dtype=out_dtype, device=workspace.device)
    if out.dtype not in (torch.float32, torch.float16) or not out.is_contiguous() or \
            out.shape != (num_seqs, num_q_heads, HEAD_DIM):
        raise ValueError("out must be contiguous fp32/fp16 [B][Hq][128]")
    st = load().kvq_decode_combine_slots(
        _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16, num_seqs, num_q_heads, _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(total_slots), int(bool(rotated)), _stream_ptr(stream))
    _check(st, "kvq_decode_combine_slots")
    return out


def slots_workspace_bytes(num_seqs: int, num_q_heads: int, total_slots: int) -> int:
    """Bytes of a slotted workspace: fp32 [B][Hq][total_slots][132]."""
    return num_seqs * num_q_heads * total_slots * 132 * 4

