"""CPU oracle for paged KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``liboracle.so`` (plain C, every
step in double precision, see ``pkv_oracle.c`` for the passages each function
follows) with numpy arguments. It shares no code with the GPU library and
imports nothing from it.

Dtype codes used here (the oracle's own): 0 float32, 1 float16, 2 bfloat16
(raw uint16 bits), 3 OCP fp8 E4M3FN (raw uint8 codes).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16, FP8 = 0, 1, 2, 3
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, FP8: 1}
BLOCK = 16

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        c_i64, c_int, c_dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = c_int
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_double.restype = c_dbl
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = c_dbl
        L.oracle_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e4m3_to_double.restype = c_dbl
        L.oracle_fp8_e4m3_encode.argtypes = [c_dbl, c_dbl]
        L.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_fp8_e4m3_encode_f32.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_fp8_e4m3_encode_f32.restype = ctypes.c_uint8
        L.oracle_kv_append_fp8.argtypes = [vp, vp, c_int, vp, c_i64, vp, vp, c_i64, c_i64, c_i64,
                                           ctypes.c_float, ctypes.c_float]
        L.oracle_kv_append_fp8.restype = c_int
        L.oracle_kv_bytes_per_token.argtypes = [c_i64, c_i64, c_i64, c_i64]
        L.oracle_kv_bytes_per_token.restype = ctypes.c_uint64
        L.oracle_kv_append.argtypes = [vp, vp, c_int, vp, c_i64, vp, vp, c_i64, c_i64, c_i64]
        L.oracle_kv_append.restype = c_int
        L.oracle_gather.argtypes = [vp, vp, c_int, c_i64, c_i64, c_i64, vp, c_i64, vp, c_i64,
                                    c_i64, vp, vp]
        L.oracle_gather.restype = c_int
        L.oracle_paged_decode.argtypes = [vp, c_int, c_i64, c_i64, vp, vp, c_int, c_dbl, c_dbl,
                                          c_i64, c_i64, c_i64, vp, c_i64, vp, c_dbl, vp]
        L.oracle_paged_decode.restype = c_int
        L.oracle_paged_decode_split.argtypes = [vp, c_int, c_i64, c_i64, vp, vp, c_int, c_dbl,
                                                c_dbl, c_i64, c_i64, c_i64, vp, c_i64, vp, c_dbl,
                                                c_i64, vp, vp, vp, vp]
        L.oracle_paged_decode_split.restype = c_int
        L.oracle_paged_prefill.argtypes = [vp, c_int, c_i64, c_i64, vp, vp, vp, c_int, c_dbl,
                                           c_dbl, c_i64, c_i64, c_i64, vp, c_i64, vp, c_dbl, vp]
        L.oracle_paged_prefill.restype = c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"oracle: unsupported storage dtype {a.dtype}")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


# ---- element codecs --------------------------------------------------------

def f16_to_double(bits: int) -> float:
    return lib().oracle_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def fp8_e4m3_to_double(code: int) -> float:
    return lib().oracle_fp8_e4m3_to_double(code)


def fp8_e4m3_encode(x: float, scale: float = 1.0) -> int:
    return lib().oracle_fp8_e4m3_encode(float(x), float(scale))


def fp8_e4m3_encode_f32(x: float, scale: float = 1.0) -> int:
    """The code of the float32 quotient x / scale (see pkv_oracle.c)."""
    return lib().oracle_fp8_e4m3_encode_f32(float(x), float(scale))


# ---- sizing ----------------------------------------------------------------

def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """2 (K and V) * L * H_kv * d * b (ttlab page, section 2)."""
    return int(lib().oracle_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes))


# ---- append / gather -------------------------------------------------------

def kv_append(k, v, slot_mapping, k_cache, v_cache):
    """In-place byte copy of each new token's rows into its slot (see pkv_oracle.c)."""
    num_blocks, H, blk, d = k_cache.shape
    assert blk == BLOCK and k.shape[1:] == (H, d) and v.shape == k.shape
    assert k.dtype == k_cache.dtype == v.dtype == v_cache.dtype
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    rc = lib().oracle_kv_append(_ptr(k), _ptr(v), _dtype_code(k), _ptr(slots), k.shape[0],
                                _ptr(k_cache), _ptr(v_cache), num_blocks, H, d)
    if rc != 0:
        raise ValueError("oracle_kv_append: slot out of range")


def kv_append_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """In-place quantising append of float32 / float16 / bfloat16 rows (bfloat16
    as uint16 bits) into uint8 E4M3FN caches (see pkv_oracle.c)."""
    num_blocks, H, blk, d = k_cache.shape
    assert blk == BLOCK and k.shape[1:] == (H, d) and v.shape == k.shape and k.dtype == v.dtype
    assert k_cache.dtype == v_cache.dtype == np.uint8
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    rc = lib().oracle_kv_append_fp8(_ptr(k), _ptr(v), _dtype_code(k), _ptr(slots), k.shape[0],
                                    _ptr(k_cache), _ptr(v_cache), num_blocks, H, d,
                                    float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError("oracle_kv_append_fp8: bad dtype or slot out of range")


def gather(k_cache, v_cache, block_tables, context_lens, max_ctx, fill=None):
    """Contiguous [S][H][max_ctx][d] copies of every sequence's K and V rows."""
    num_blocks, H, blk, d = k_cache.shape
    S = context_lens.shape[0]
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    k_out = np.zeros((S, H, max_ctx, d), dtype=k_cache.dtype)
    v_out = np.zeros((S, H, max_ctx, d), dtype=k_cache.dtype)
    if fill is not None:
        k_out.view(np.uint8)[...] = fill
        v_out.view(np.uint8)[...] = fill
    rc = lib().oracle_gather(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), num_blocks, H, d,
                             _ptr(bt), bt.shape[1], _ptr(cl), S, max_ctx, _ptr(k_out),
                             _ptr(v_out))
    if rc != 0:
        raise ValueError("oracle_gather: block id out of range")
    return k_out, v_out


# ---- decode ----------------------------------------------------------------

def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0):
    """Paged decode attention in double precision; returns out [S][H_q][d] float64."""
    S, Hq, d = q.shape
    num_blocks, H, blk, d2 = k_cache.shape
    assert blk == BLOCK and d2 == d and v_cache.shape == k_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty((S, Hq, d), dtype=np.float64)
    rc = lib().oracle_paged_decode(_ptr(q), _dtype_code(q), S, Hq, _ptr(k_cache), _ptr(v_cache),
                                   _dtype_code(k_cache), k_scale, v_scale, num_blocks, H, d,
                                   _ptr(bt), bt.shape[1], _ptr(cl), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_paged_decode: invalid arguments")
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                  k_scale=1.0, v_scale=1.0):
    """Paged chunked-prefill attention in double precision (see
    pkv_oracle.c): q is [T][H_q][d] with sequence s owning rows
    [query_start[s], query_start[s + 1]); returns out [T][H_q][d] float64."""
    T, Hq, d = q.shape
    num_blocks, H, blk, d2 = k_cache.shape
    assert blk == BLOCK and d2 == d and v_cache.shape == k_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    S = cl.shape[0]
    assert qs.shape == (S + 1,) and qs[-1] == T
    out = np.empty((T, Hq, d), dtype=np.float64)
    rc = lib().oracle_paged_prefill(_ptr(q), _dtype_code(q), S, Hq, _ptr(qs), _ptr(k_cache),
                                    _ptr(v_cache), _dtype_code(k_cache), k_scale, v_scale,
                                    num_blocks, H, d, _ptr(bt), bt.shape[1], _ptr(cl),
                                    float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_paged_prefill: invalid arguments")
    return out


def paged_decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                       k_scale=1.0, v_scale=1.0):
    """Split-KV form: returns (out, part_m, part_l, part_o), all float64."""
    S, Hq, d = q.shape
    num_blocks, H, blk, d2 = k_cache.shape
    assert blk == BLOCK and d2 == d
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    pn = (bt.shape[1] * BLOCK + partition_size - 1) // partition_size
    pm = np.empty((S, Hq, pn), dtype=np.float64)
    pl = np.empty((S, Hq, pn), dtype=np.float64)
    po = np.empty((S, Hq, pn, d), dtype=np.float64)
    out = np.empty((S, Hq, d), dtype=np.float64)
    rc = lib().oracle_paged_decode_split(_ptr(q), _dtype_code(q), S, Hq, _ptr(k_cache),
                                         _ptr(v_cache), _dtype_code(k_cache), k_scale, v_scale,
                                         num_blocks, H, d, _ptr(bt), bt.shape[1], _ptr(cl),
                                         float(scale), partition_size, _ptr(pm), _ptr(pl),
                                         _ptr(po), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_paged_decode_split: invalid arguments")
    return out, pm, pl, po
