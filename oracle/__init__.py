"""CPU oracle for the K4V2 group-128 KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
``kvq_oracle.c``) with numpy marshalling and holds no arithmetic of its own.
The GPU library never imports it and shares no code with it.

Functions and the passages they follow (pages cited by title and section):

* ``quantize_group`` / ``quantize_append`` -- the KVarN write path: Hadamard
  rotation, variance normalisation, asymmetric round-to-nearest (dothoosh.com,
  "KVarN vs TurboQuant: 5x more context with higher accuracy", the four-stage
  pipeline list, stages 1-3; beyondheadline.xyz, "Huawei's KV-cache trick",
  section "The claim that breaks the usual trade-off": 4-bit keys, 2-bit
  values, cache blocks, preset kvarn_k4v2_g128).
* ``decode_attention`` -- attention over the dequantised, un-rotated cache by
  its plain definition (softmax(scale q.k) v), fp64.
* ``decode_attention_folded`` -- the same result reached by scale folding on
  read-back (same pipeline list, stage 4), fp64; pins the algebra.
* ``decode_attention_mq`` -- several causal query rows per sequence (the
  multi-token decode of speculative drafts and prefill chunks), fp64.
* ``page_tokens`` -- pages of 16, 32, 64 or 128 tokens, each (page, KV head)
  made of page_tokens / 16 consecutive 16-token regions (the variable page
  size the dothoosh.com page announces in its closing list).
* ``fmt=(kbits, vbits)`` -- the same pipeline at the other bit widths the pages
  report (8-bit keys with 4-bit values, 4-bit both, and 3-bit codes: dzen.ru
  summary of the vLLM TurboQuant post, sections on accuracy and memory); keys
  4 or 8 bits with values 2 or 4 bits, or 3 bits both (stored as bit
  planes).  The default (4, 2) is the KVarN preset.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

D = 128
PAGE = 16
REGION = 1664

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.kvqo_half_to_double.argtypes = [ctypes.c_uint16]
    lib.kvqo_half_to_double.restype = ctypes.c_double
    lib.kvqo_float_to_half.argtypes = [ctypes.c_float]
    lib.kvqo_float_to_half.restype = ctypes.c_uint16
    lib.kvqo_hadamard_entry.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.kvqo_hadamard_entry.restype = ctypes.c_int
    lib.kvqo_fwht_f32.argtypes = [P]
    lib.kvqo_fwht_f32.restype = None
    lib.kvqo_hadamard_matvec_f64.argtypes = [P, P]
    lib.kvqo_hadamard_matvec_f64.restype = None
    lib.kvqo_quantize_group_mode.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
    lib.kvqo_quantize_group_mode.restype = None
    lib.kvqo_attention_f16.argtypes = [P, P, i64, P, i32, ctypes.c_double, P]
    lib.kvqo_attention_f16.restype = None
    lib.kvqo_attention_f64.argtypes = [P, P, i64, P, i32, ctypes.c_double, P]
    lib.kvqo_attention_f64.restype = None
    ci = ctypes.c_int
    lib.kvqo_region_bytes.argtypes = [ci, ci]
    lib.kvqo_region_bytes.restype = i64
    lib.kvqo_store_token_fmt.argtypes = [ci, ci, P, ci, P, ctypes.c_uint16, ctypes.c_uint16,
                                         P, ctypes.c_uint16, ctypes.c_uint16]
    lib.kvqo_store_token_fmt.restype = None
    lib.kvqo_load_token_fmt.argtypes = [ci, ci, P, ci, P, P, P, P, P, P]
    lib.kvqo_load_token_fmt.restype = None
    lib.kvqo_dequant_slot_fmt.argtypes = [ci, ci, P, ci, P, P]
    lib.kvqo_dequant_slot_fmt.restype = None
    lib.kvqo_dequant_slot_rotated_fmt.argtypes = [ci, ci, P, ci, P, P]
    lib.kvqo_dequant_slot_rotated_fmt.restype = None
    lib.kvqo_decode_attention_folded_fmt.argtypes = [ci, ci, P, i64, i32, P, i32, P, i32, i32, P,
                                                     ctypes.c_double, P]
    lib.kvqo_decode_attention_folded_fmt.restype = ctypes.c_int
    lib.kvqo_quantize_append_paged.argtypes = [ci, ci, ci, P, P, i64, i64, P, i64, i32, P, i64]
    lib.kvqo_quantize_append_paged.restype = ctypes.c_int
    lib.kvqo_decode_attention_paged.argtypes = [ci, ci, ci, P, i64, i32, P, i32, P, i32, i32, P,
                                                ctypes.c_double, P, P]
    lib.kvqo_decode_attention_paged.restype = ctypes.c_int
    lib.kvqo_decode_attention_mq_paged.argtypes = [ci, ci, ci, P, i64, i32, P, i32, P, i32, i32, i32, P,
                                                   ctypes.c_double, P]
    lib.kvqo_decode_attention_mq_paged.restype = ctypes.c_int
    lib.kvqo_block_variant.argtypes = [P, P, ci, ci, ci, P, P, P, P, P]
    lib.kvqo_block_variant.restype = ci
    lib.kvqo_quantize_append_pb.argtypes = [P, P, i64, i64, P, i64, i32, P, i64]
    lib.kvqo_quantize_append_pb.restype = ci
    lib.kvqo_dequant_slot_pb.argtypes = [P, ci, P, P]
    lib.kvqo_dequant_slot_pb.restype = None
    lib.kvqo_decode_attention_pb.argtypes = [P, i64, i32, P, i32, P, i32, i32, P, ctypes.c_double, P, P]
    lib.kvqo_decode_attention_pb.restype = ci
    lib.kvqo_pb_region_bytes.argtypes = []
    lib.kvqo_pb_region_bytes.restype = ci
    lib.kvqo_pb_iters.argtypes = []
    lib.kvqo_pb_iters.restype = ci
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def half_to_double(bits: int) -> float:
    return _load().kvqo_half_to_double(int(bits) & 0xFFFF)


def float_to_half(x: float) -> int:
    return int(_load().kvqo_float_to_half(float(np.float32(x))))


def hadamard_entry(i: int, j: int) -> int:
    return _load().kvqo_hadamard_entry(i, j)


def fwht_f32(x: np.ndarray) -> np.ndarray:
    y = _c(x, np.float32).copy()
    assert y.shape == (D,)
    _load().kvqo_fwht_f32(_ptr(y))
    return y


def hadamard_matvec_f64(x: np.ndarray) -> np.ndarray:
    xx = _c(x, np.float64)
    y = np.empty(D, np.float64)
    _load().kvqo_hadamard_matvec_f64(_ptr(xx), _ptr(y))
    return y


def quantize_group(x_f16: np.ndarray, bits: int, offset_mode: int | None = None):
    """x_f16: 128 float16 values.  Returns (codes uint8[128], s_bits, offset_bits);
    the offset is the zero z (keys, offset_mode 0) or the group mean mu
    (values, offset_mode 1).  By default 4-bit groups are keys, 2-bit values."""
    x = _c(x_f16, np.float16).view(np.uint16)
    assert x.shape == (D,)
    if offset_mode is None:
        offset_mode = 1 if bits == 2 else 0
    codes = np.empty(D, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    _load().kvqo_quantize_group_mode(_ptr(x), int(bits), int(offset_mode), _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


def group_zero(codes: np.ndarray, s_bits: int, off_bits: int, is_value: bool) -> float:
    """Rotated-domain zero-point of a group: z (keys) or mu - s*C/128 (values)."""
    off = half_to_double(off_bits)
    if not is_value:
        return off
    return off - half_to_double(s_bits) * int(np.sum(codes, dtype=np.int64)) / 128.0


K4V2 = (4, 2)


def region_bytes(fmt=K4V2) -> int:
    """Bytes of one (page, KV head) region for (kbits, vbits)."""
    n = int(_load().kvqo_region_bytes(int(fmt[0]), int(fmt[1])))
    if n <= 0:
        raise ValueError(f"unsupported bit widths {fmt}")
    return n


def store_token(region: np.ndarray, off: int, kc, ks, kz, vc, vs, vz, fmt=K4V2):
    assert region.dtype == np.uint8 and region.size == region_bytes(fmt) and region.flags.c_contiguous
    _load().kvqo_store_token_fmt(int(fmt[0]), int(fmt[1]), _ptr(region), int(off), _ptr(_c(kc, np.uint8)),
                                 int(ks), int(kz), _ptr(_c(vc, np.uint8)), int(vs), int(vz))


def load_token(region: np.ndarray, off: int, fmt=K4V2):
    r = _c(region, np.uint8)
    assert r.size == region_bytes(fmt)
    kc = np.empty(D, np.uint8)
    vc = np.empty(D, np.uint8)
    m = np.zeros(4, np.uint16)
    _load().kvqo_load_token_fmt(int(fmt[0]), int(fmt[1]), _ptr(r), int(off), _ptr(kc), _ptr(m[0:1]),
                                _ptr(m[1:2]), _ptr(vc), _ptr(m[2:3]), _ptr(m[3:4]))
    return kc, int(m[0]), int(m[1]), vc, int(m[2]), int(m[3])


def quantize_append(key_f16: np.ndarray, value_f16: np.ndarray, slot_mapping: np.ndarray,
                    pool: np.ndarray, fmt=K4V2, page_tokens: int = PAGE) -> None:
    """key/value: float16 [T][Hkv][128]; slot_mapping int64[T] (page *
    page_tokens + offset); pool uint8 [num_pages][Hkv][page_tokens / 16 *
    region_bytes(fmt)], written in place."""
    k = _c(key_f16, np.float16)
    v = _c(value_f16, np.float16)
    T, H, d = k.shape
    assert d == D and v.shape == k.shape
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    assert pool.shape[1:] == (H, page_tokens // PAGE * region_bytes(fmt))
    sm = _c(slot_mapping, np.int64)
    rc = _load().kvqo_quantize_append_paged(int(fmt[0]), int(fmt[1]), int(page_tokens), _ptr(k), _ptr(v), H * D,
                                            H * D, _ptr(sm), T, H, _ptr(pool), pool.shape[0])
    if rc != 0:
        raise ValueError("oracle append: slot outside the pool")


def dequant_slot(region: np.ndarray, off: int, fmt=K4V2):
    r = _c(region, np.uint8)
    k = np.empty(D, np.float64)
    v = np.empty(D, np.float64)
    _load().kvqo_dequant_slot_fmt(int(fmt[0]), int(fmt[1]), _ptr(r), int(off), _ptr(k), _ptr(v))
    return k, v


def dequant_slot_rotated(region: np.ndarray, off: int, fmt=K4V2):
    r = _c(region, np.uint8)
    k = np.empty(D, np.float64)
    v = np.empty(D, np.float64)
    _load().kvqo_dequant_slot_rotated_fmt(int(fmt[0]), int(fmt[1]), _ptr(r), int(off), _ptr(k), _ptr(v))
    return k, v


def decode_attention(pool, block_tables, seq_lens, query_f16, scale, head_mask=None, fmt=K4V2,
                     page_tokens: int = PAGE):
    """Plain-definition decode attention in fp64.  query: float16 [B][Hq][128].
    Returns float64 [B][Hq][128] (NaN where head_mask excludes a head)."""
    pool = _c(pool, np.uint8)
    assert pool.shape[2] == page_tokens // PAGE * region_bytes(fmt)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    q = _c(query_f16, np.float16)
    B, Hq, d = q.shape
    Hkv = pool.shape[1]
    out = np.full((B, Hq, D), np.nan, np.float64)
    hm = None if head_mask is None else _c(head_mask, np.uint8)
    rc = _load().kvqo_decode_attention_paged(int(fmt[0]), int(fmt[1]), int(page_tokens), _ptr(pool), pool.shape[0],
                                             Hkv, _ptr(bt), bt.shape[1], _ptr(sl), B, Hq, _ptr(q), float(scale),
                                             None if hm is None else _ptr(hm), _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode: invalid shape or page id")
    return out


def decode_attention_mq(pool, block_tables, seq_lens, query_f16, scale, fmt=K4V2, page_tokens: int = PAGE):
    """Several query rows per sequence, causal: query float16 [B][M][Hq][128];
    row m of sequence b attends to tokens 0 .. seq_lens[b] - M + m.  Returns
    float64 [B][M][Hq][128]."""
    pool = _c(pool, np.uint8)
    assert pool.shape[2] == page_tokens // PAGE * region_bytes(fmt)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    q = _c(query_f16, np.float16)
    B, M, Hq, d = q.shape
    out = np.empty((B, M, Hq, D), np.float64)
    rc = _load().kvqo_decode_attention_mq_paged(int(fmt[0]), int(fmt[1]), int(page_tokens), _ptr(pool),
                                                pool.shape[0], pool.shape[1], _ptr(bt), bt.shape[1], _ptr(sl), B, M,
                                                Hq, _ptr(q), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle multi-query decode: invalid shape or page id")
    return out


def decode_attention_folded(pool, block_tables, seq_lens, query_f16, scale, fmt=K4V2):
    pool = _c(pool, np.uint8)
    assert pool.shape[2] == region_bytes(fmt)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    q = _c(query_f16, np.float16)
    B, Hq, d = q.shape
    out = np.empty((B, Hq, D), np.float64)
    rc = _load().kvqo_decode_attention_folded_fmt(int(fmt[0]), int(fmt[1]), _ptr(pool), pool.shape[0],
                                                  pool.shape[1], _ptr(bt), bt.shape[1], _ptr(sl), B, Hq,
                                                  _ptr(q), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle folded decode: invalid shape or page id")
    return out


def attention_f16(k_f16, v_f16, q_f16, scale):
    """Plain fp64 attention of G query heads over fp16 tokens of one KV head:
    k, v float16 [n][128], q float16 [G][128] -> float64 [G][128]."""
    k = _c(k_f16, np.float16)
    v = _c(v_f16, np.float16)
    q = _c(q_f16, np.float16)
    n = k.shape[0]
    assert v.shape == k.shape and k.shape[1:] == (D,) and q.shape[1:] == (D,)
    out = np.empty((q.shape[0], D), np.float64)
    _load().kvqo_attention_f16(_ptr(k), _ptr(v), n, _ptr(q), q.shape[0], float(scale), _ptr(out))
    return out


def attention_f64(k, v, q_f16, scale):
    """Plain fp64 attention of G query heads over tokens given in fp64:
    k, v [n][128], q float16 [G][128] -> float64 [G][128]."""
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    q = _c(q_f16, np.float16)
    assert v.shape == k.shape and k.shape[1:] == (D,) and q.shape[1:] == (D,)
    out = np.empty((q.shape[0], D), np.float64)
    _load().kvqo_attention_f64(_ptr(k), _ptr(v), k.shape[0], _ptr(q), q.shape[0], float(scale), _ptr(out))
    return out



def block_variant(x_f16, bits: int, iters: int, present=None):
    """Page-balanced variance normalisation of one block of T <= 16 tokens
    (kvqo_block_variant): x float16 [T][128] -> (codes uint8 [T][128], the
    rebuilt original-domain block float64 [T][128], s and z fp16 bits [T],
    column exponents int [128]).  iters = number of column passes (0: the
    per-token encoder); present (optional bool [T]) marks absent rows."""
    x = _c(x_f16, np.float16)
    T = x.shape[0]
    assert x.shape == (T, D) and T <= PAGE
    codes = np.zeros((T, D), np.uint8)
    out = np.zeros((T, D), np.float64)
    s = np.zeros(T, np.uint16)
    z = np.zeros(T, np.uint16)
    e = np.zeros(D, np.int32)
    pres = None if present is None else _c(np.asarray(present, np.uint8), np.uint8)
    rc = _load().kvqo_block_variant(_ptr(x.view(np.uint16)), None if pres is None else _ptr(pres), T, int(bits),
                                    int(iters), _ptr(codes), _ptr(s), _ptr(z), _ptr(e), _ptr(out))
    if rc != 0:
        raise ValueError("block_variant: invalid arguments")
    return codes, out, s, z, e


# The page-balanced key preset (kvqo_quantize_append_pb): K4V2 regions followed
# by 128 column-scale bytes.
PB_REGION = 1792


def pb_iters() -> int:
    return int(_load().kvqo_pb_iters())


def pb_region_bytes() -> int:
    return int(_load().kvqo_pb_region_bytes())


def quantize_append_pb(key_f16: np.ndarray, value_f16: np.ndarray, slot_mapping: np.ndarray, pool: np.ndarray) -> int:
    """Whole-page append into a page-balanced pool u8 [num_pages][H][1792]:
    call tokens 16b..16b+15 fill page slot_mapping[16b] / 16 from slot 0."""
    k = _c(key_f16, np.float16)
    v = _c(value_f16, np.float16)
    T, H, _ = k.shape
    assert v.shape == k.shape and pool.dtype == np.uint8 and pool.shape[1:] == (H, PB_REGION)
    assert pool.flags.c_contiguous
    sm = _c(slot_mapping, np.int64)
    return int(_load().kvqo_quantize_append_pb(_ptr(k.view(np.uint16)), _ptr(v.view(np.uint16)), H * D, H * D,
                                               _ptr(sm), T, H, _ptr(pool), pool.shape[0]))


def dequant_slot_pb(region: np.ndarray, off: int):
    assert region.dtype == np.uint8 and region.size == PB_REGION and region.flags.c_contiguous
    k = np.empty(D, np.float64)
    v = np.empty(D, np.float64)
    _load().kvqo_dequant_slot_pb(_ptr(region), int(off), _ptr(k), _ptr(v))
    return k, v


def decode_attention_pb(pool, block_tables, seq_lens, query_f16, scale, head_mask=None):
    """Plain fp64 decode over a page-balanced pool (16-token pages)."""
    assert pool.dtype == np.uint8 and pool.shape[2] == PB_REGION and pool.flags.c_contiguous
    bt = _c(block_tables, np.int32)
    lens = _c(seq_lens, np.int32)
    q = _c(query_f16, np.float16)
    B, Hq, _ = q.shape
    out = np.zeros((B, Hq, D), np.float64)
    hm = None if head_mask is None else _c(head_mask, np.uint8)
    rc = _load().kvqo_decode_attention_pb(_ptr(pool), pool.shape[0], pool.shape[1], _ptr(bt), bt.shape[1],
                                          _ptr(lens), B, Hq, _ptr(q.view(np.uint16)), float(scale),
                                          None if hm is None else _ptr(hm), _ptr(out))
    if rc != 0:
        raise ValueError("decode_attention_pb: invalid shape or page id")
    return out
