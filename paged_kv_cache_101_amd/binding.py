"""Thin ctypes binding of libpkv.so (include/pkv.h).

Argument marshalling only: torch tensors in, raw device pointers, dtype codes
and sizes out to the C entry points of the same names; every step of the
computation runs in the HIP kernels behind them. Shapes, dtypes and
contiguity are checked here so that a wrong call fails with a Python error
before reaching the library. Without a built library every call raises: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_ERR_TOO_LARGE = -5

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
PKV_BLOCK_SIZE = 16
PKV_MAX_WORKERS = 4096
PKV_NOALLOC_SCRATCH_BYTES = 48 << 20

DTYPE_CODES = {"f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3}
_TORCH_CODES = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}

EXPORTS = ("pkv_status_string", "pkv_kv_bytes_per_token", "pkv_cache_tensor_bytes",
           "pkv_kv_append", "pkv_decode_workspace_bytes", "pkv_paged_attention_decode",
           "pkv_shared_prefix_workspace_bytes", "pkv_paged_attention_decode_shared_prefix",
           "pkv_paged_attention_prefill", "pkv_prefill_workspace_bytes", "pkv_copy_blocks",
           "pkv_debug_gather", "pkv_paged_attention_decode_noalloc", "pkv_stream_read",
           # host block manager (pkv_blocks.h; bound in blocks.py)
           "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_num_free_blocks", "pkv_bm_add_request",
           "pkv_bm_can_append", "pkv_bm_append", "pkv_bm_fork", "pkv_bm_free_request",
           "pkv_bm_num_tokens", "pkv_bm_num_blocks", "pkv_bm_ref_count", "pkv_bm_block_tables",
           "pkv_bm_prefix_groups", "pkv_bm_prefix_cache_stats")


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


class pkv_cache_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


_lib = None


def lib():
    """The loaded libpkv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpkv.so not found at {LIB_PATH}: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_size_t, ctypes.c_float)
        descp = ctypes.POINTER(pkv_cache_desc)
        L.pkv_status_string.argtypes = [ctypes.c_int]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_kv_bytes_per_token.argtypes = [i32, i32, i32, i32]
        L.pkv_kv_bytes_per_token.restype = sz
        L.pkv_cache_tensor_bytes.argtypes = [descp]
        L.pkv_cache_tensor_bytes.restype = sz
        L.pkv_kv_append.argtypes = [vp, vp, i32, vp, i32, vp, vp, descp, vp]
        L.pkv_kv_append.restype = ctypes.c_int
        L.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.pkv_decode_workspace_bytes.restype = sz
        L.pkv_paged_attention_decode.argtypes = [vp, i32, i32, i32, vp, vp, descp, vp, i32, vp,
                                                 f32, i32, i32, vp, sz, vp, vp]
        L.pkv_paged_attention_decode.restype = ctypes.c_int
        L.pkv_stream_read.argtypes = [vp, sz, vp, i32, vp]
        L.pkv_stream_read.restype = ctypes.c_int
        L.pkv_paged_attention_decode_noalloc.argtypes = [vp, i32, i32, i32, vp, vp, descp, vp,
                                                         i32, vp, f32, i32, i32, vp, vp]
        L.pkv_paged_attention_decode_noalloc.restype = ctypes.c_int
        L.pkv_shared_prefix_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.pkv_shared_prefix_workspace_bytes.restype = sz
        L.pkv_paged_attention_decode_shared_prefix.argtypes = [
            vp, i32, i32, i32, vp, vp, descp, vp, i32, vp, i32, vp, vp, f32, i32, vp, sz, vp, vp]
        L.pkv_paged_attention_decode_shared_prefix.restype = ctypes.c_int
        L.pkv_paged_attention_prefill.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, descp, vp,
                                                  i32, vp, f32, vp, sz, vp, vp]
        L.pkv_paged_attention_prefill.restype = ctypes.c_int
        L.pkv_prefill_workspace_bytes.argtypes = [i32]
        L.pkv_prefill_workspace_bytes.restype = sz
        L.pkv_copy_blocks.argtypes = [vp, vp, descp, vp, i32, vp]
        L.pkv_copy_blocks.restype = ctypes.c_int
        L.pkv_debug_gather.argtypes = [vp, vp, descp, vp, i32, vp, i32, i32, vp, vp, vp]
        L.pkv_debug_gather.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def _check(fn: str, rc: int):
    if rc != PKV_OK:
        raise PkvError(fn, rc)


def _ptr(t: Optional[torch.Tensor]):
    # a plain int: the argtypes (c_void_p) convert it without a wrapper object
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    """The stream handle: the given torch stream's, or the current stream of
    the current device, read directly rather than through a Stream object.
    With plain int pointers this took a decode call's host cost from 10.5 to
    7.4 us (the bare C call: 3.9 us), which matters when a step is dozens of
    short launches."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
    return stream.cuda_stream


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def cache_desc(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
               k_scale: float = 1.0, v_scale: float = 1.0) -> pkv_cache_desc:
    return pkv_cache_desc(num_blocks, PKV_BLOCK_SIZE, num_kv_heads, head_dim, DTYPE_CODES[dtype],
                          k_scale, v_scale)


def desc_for(k_cache: torch.Tensor, dtype: str, k_scale=1.0, v_scale=1.0) -> pkv_cache_desc:
    nb, H, bs, d = k_cache.shape
    _need(bs == PKV_BLOCK_SIZE, "cache must be [num_blocks][H_kv][16][head_dim]")
    return cache_desc(nb, H, d, dtype, k_scale, v_scale)


def _dtype_of(t: torch.Tensor, declared: Optional[str] = None) -> int:
    if t.dtype == torch.uint8:
        _need(declared in (None, "fp8"), "uint8 tensors hold fp8 E4M3 codes")
        return PKV_FP8_E4M3
    if t.dtype == torch.float8_e4m3fn:
        return PKV_FP8_E4M3
    _need(t.dtype in _TORCH_CODES, f"unsupported tensor dtype {t.dtype}")
    return _TORCH_CODES[t.dtype]


# bytes per element of each dtype code (pkv_dtype)
_ELEM_BYTES = {PKV_F32: 4, PKV_F16: 2, PKV_BF16: 2, PKV_FP8_E4M3: 1}


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_desc_caches(desc: pkv_cache_desc, k_cache: torch.Tensor, v_cache: torch.Tensor):
    """The caches must hold the pool the descriptor describes (the C side
    cannot see tensor sizes, so a descriptor larger than the tensors would
    make the kernels read or write past their ends)."""
    eb = _ELEM_BYTES.get(desc.dtype)
    _need(eb is not None, f"descriptor dtype {desc.dtype} unknown")
    need = desc.num_blocks * desc.num_kv_heads * PKV_BLOCK_SIZE * desc.head_dim * eb
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(_nbytes(t) >= need,
              f"{name} holds {_nbytes(t)} bytes, the descriptor's pool needs {need}")
        _need(_dtype_of(t, "fp8" if desc.dtype == PKV_FP8_E4M3 else None) == desc.dtype
              or (desc.dtype == PKV_FP8_E4M3 and t.dtype == torch.uint8),
              f"{name} dtype {t.dtype} does not match the descriptor")


def _check_rows(name: str, t: torch.Tensor, desc: pkv_cache_desc, heads: Optional[int] = None):
    """t: [rows][heads][desc.head_dim]; heads a multiple of desc.num_kv_heads
    (query heads, at most 8 per KV head) unless given exactly."""
    _need(t.dim() == 3, f"{name} must be [rows][heads][head_dim]")
    _need(t.shape[2] == desc.head_dim,
          f"{name} head_dim {t.shape[2]} != descriptor head_dim {desc.head_dim}")
    if heads is not None:
        _need(t.shape[1] == heads, f"{name} has {t.shape[1]} heads, expected {heads}")
    else:
        _need(t.shape[1] % desc.num_kv_heads == 0,
              f"{name} heads {t.shape[1]} not a multiple of num_kv_heads {desc.num_kv_heads}")


def _check_device(*ts):
    for t in ts:
        _need(t.is_contiguous() and t.is_cuda, "all tensors must be contiguous device tensors")


def _no_capture(what: str):
    """Allocating a workspace from torch inside a graph capture would record a
    memset into the graph: the caller must pass one made beforehand."""
    if torch.cuda.is_available() and torch.cuda.is_current_stream_capturing():
        raise RuntimeError(f"{what}: pass a workspace made before the graph capture "
                           "(allocating one here would capture a memset)")


# ---- entry points (same names as the C ABI) --------------------------------

def pkv_kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype: str) -> int:
    return int(lib().pkv_kv_bytes_per_token(num_layers, num_kv_heads, head_dim,
                                            DTYPE_CODES[dtype]))


def pkv_cache_tensor_bytes(desc: pkv_cache_desc) -> int:
    return int(lib().pkv_cache_tensor_bytes(ctypes.byref(desc)))


def pkv_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                               head_dim: int, max_blocks_per_seq: int = 1,
                               partition_size: int = 0, num_workers: int = 0) -> int:
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_blocks_per_seq, partition_size, num_workers))


def decode_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     num_workers: int = 0, device=None, max_blocks_per_seq: int = 1,
                     partition_size: int = 0) -> torch.Tensor:
    """A zero-filled decode workspace (its counters must start at zero; every
    decode call leaves them zero, so it can be reused call after call)."""
    n = pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   max_blocks_per_seq, partition_size, num_workers)
    _need(n > 0, "invalid decode shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pkv_kv_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, desc: pkv_cache_desc,
                  stream=None) -> None:
    """k, v: [T][H_kv][d] in the cache dtype, or float32 / float16 / bfloat16
    rows into an fp8 cache (quantised with desc.k_scale / desc.v_scale);
    slot_mapping: int64 [T]."""
    T = k.shape[0]
    _need(k.shape == v.shape and k.dim() == 3, "k and v must be [T][H_kv][d]")
    _check_rows("k", k, desc, heads=desc.num_kv_heads)
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T,
          "slot_mapping must be int64 [T]")
    _need(k.dtype == v.dtype and k_cache.dtype == v_cache.dtype, "k/v or cache dtypes differ")
    _need(k.dtype == k_cache.dtype
          or (_dtype_of(k_cache, "fp8") == PKV_FP8_E4M3 and _dtype_of(k) != PKV_FP8_E4M3),
          "k/v must be in the cache dtype, or 16/32-bit floats into an fp8 cache")
    _check_desc_caches(desc, k_cache, v_cache)
    _check_device(k, v, slot_mapping, k_cache, v_cache)
    rc = lib().pkv_kv_append(_ptr(k), _ptr(v), _dtype_of(k), _ptr(slot_mapping), T,
                             _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _stream(stream))
    _check("pkv_kv_append", rc)


def _check_decode_args(q, k_cache, v_cache, desc, block_tables, context_lens, out):
    S, Hq, d = q.shape
    _check_rows("q", q, desc)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == S,
          "context_lens must be int32 [S]")
    _check_desc_caches(desc, k_cache, v_cache)
    _check_device(q, k_cache, v_cache, block_tables, context_lens, out)


def pkv_paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               desc: pkv_cache_desc, block_tables: torch.Tensor,
                               context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                               num_workers: int = 0,
                               workspace: Optional[torch.Tensor] = None, stream=None,
                               partition_size: int = 0) -> None:
    """q, out: [S][H_q][d]; block_tables: int32 [S][max_blocks]; context_lens: int32 [S].
    partition_size: 0 (balanced split) or tokens per fixed partition.
    A zero-filled workspace (decode_workspace) is allocated from torch when
    none is given (not allowed while a graph is being captured)."""
    _check_decode_args(q, k_cache, v_cache, desc, block_tables, context_lens, out)
    S, Hq, d = q.shape
    mb = block_tables.shape[1]
    if workspace is None:
        _no_capture("pkv_paged_attention_decode")
        workspace = decode_workspace(S, Hq, desc.num_kv_heads, d, num_workers, q.device, mb,
                                     partition_size)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a device tensor")
    rc = lib().pkv_paged_attention_decode(
        _ptr(q), _dtype_of(q), S, Hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
        _ptr(block_tables), mb, _ptr(context_lens), float(scale), partition_size, num_workers,
        _ptr(workspace), _nbytes(workspace), _ptr(out), _stream(stream))
    _check("pkv_paged_attention_decode", rc)


def pkv_paged_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                       v_cache: torch.Tensor, desc: pkv_cache_desc,
                                       block_tables: torch.Tensor, context_lens: torch.Tensor,
                                       scale: float, out: torch.Tensor, num_workers: int = 0,
                                       stream=None, partition_size: int = 0) -> None:
    """pkv_paged_attention_decode with the library's static scratch as its
    workspace: nothing is allocated, here or in the library (for graph
    capture and loops that must not allocate). Calls that overlap on one GPU
    share that scratch and race."""
    _check_decode_args(q, k_cache, v_cache, desc, block_tables, context_lens, out)
    S, Hq, d = q.shape
    rc = lib().pkv_paged_attention_decode_noalloc(
        _ptr(q), _dtype_of(q), S, Hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), float(scale),
        partition_size, num_workers, _ptr(out), _stream(stream))
    _check("pkv_paged_attention_decode_noalloc", rc)


def pkv_shared_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                      head_dim: int, num_groups: int, num_workers: int = 0) -> int:
    return int(lib().pkv_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, num_groups, num_workers))


def shared_prefix_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            num_groups: int, num_workers: int = 0, device=None) -> torch.Tensor:
    """A zero-filled shared-prefix decode workspace (reusable call after call)."""
    n = pkv_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          num_groups, num_workers)
    _need(n > 0, "invalid shared-prefix decode shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pkv_paged_attention_decode_shared_prefix(
        q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, desc: pkv_cache_desc,
        block_tables: torch.Tensor, context_lens: torch.Tensor, group_starts: torch.Tensor,
        group_prefix_blocks: torch.Tensor, scale: float, out: torch.Tensor, num_workers: int = 0,
        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """As pkv_paged_attention_decode, plus prefix groups: group_starts int32
    [G + 1] and group_prefix_blocks int32 [G] (device); group j is sequences
    [group_starts[j], group_starts[j + 1]) sharing their first
    group_prefix_blocks[j] blocks."""
    _check_decode_args(q, k_cache, v_cache, desc, block_tables, context_lens, out)
    S, Hq, d = q.shape
    ng = group_prefix_blocks.numel()
    _need(group_starts.dtype == torch.int32 and group_prefix_blocks.dtype == torch.int32
          and group_starts.numel() == ng + 1, "group arrays must be int32 [G + 1] and [G]")
    _check_device(group_starts, group_prefix_blocks)
    mb = block_tables.shape[1]
    if workspace is None:
        _no_capture("pkv_paged_attention_decode_shared_prefix")
        workspace = shared_prefix_workspace(S, Hq, desc.num_kv_heads, d, ng, num_workers,
                                            q.device)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a device tensor")
    rc = lib().pkv_paged_attention_decode_shared_prefix(
        _ptr(q), _dtype_of(q), S, Hq, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
        _ptr(block_tables), mb, _ptr(context_lens), ng, _ptr(group_starts),
        _ptr(group_prefix_blocks), float(scale), num_workers, _ptr(workspace), _nbytes(workspace),
        _ptr(out), _stream(stream))
    _check("pkv_paged_attention_decode_shared_prefix", rc)


def pkv_prefill_workspace_bytes(head_dim: int) -> int:
    return int(lib().pkv_prefill_workspace_bytes(head_dim))


def prefill_workspace(head_dim: int, device=None) -> torch.Tensor:
    """A workspace that lets pkv_paged_attention_prefill split the keys of
    batches with few query rows over several workgroups."""
    n = pkv_prefill_workspace_bytes(head_dim)
    _need(n > 0, "head_dim must be 64 or 128")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pkv_paged_attention_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                desc: pkv_cache_desc, block_tables: torch.Tensor,
                                context_lens: torch.Tensor, query_start: torch.Tensor,
                                scale: float, out: torch.Tensor,
                                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """q, out: [T][H_q][d]; query_start: int32 [S + 1] (sequence s owns rows
    [query_start[s], query_start[s + 1])); block_tables, context_lens as for decode.
    workspace: None, or prefill_workspace(d) to let few-row batches split their keys."""
    T, Hq, d = q.shape
    S = context_lens.numel()
    _check_rows("q", q, desc)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(query_start.dtype == torch.int32 and query_start.numel() == S + 1,
          "query_start must be int32 [S + 1]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    _check_desc_caches(desc, k_cache, v_cache)
    _check_device(q, k_cache, v_cache, block_tables, context_lens, query_start, out)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a device tensor")
        ws_ptr, ws_bytes = _ptr(workspace), _nbytes(workspace)
    rc = lib().pkv_paged_attention_prefill(
        _ptr(q), _dtype_of(q), S, T, Hq, _ptr(query_start), _ptr(k_cache), _ptr(v_cache),
        ctypes.byref(desc), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        float(scale), ws_ptr, ws_bytes, _ptr(out), _stream(stream))
    _check("pkv_paged_attention_prefill", rc)


def pkv_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, desc: pkv_cache_desc,
                    pairs: torch.Tensor, stream=None) -> None:
    """pairs: int32 [n][2] (device) of (source block, destination block)."""
    _need(pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2,
          "pairs must be int32 [n][2]")
    _check_desc_caches(desc, k_cache, v_cache)
    _check_device(k_cache, v_cache, pairs)
    rc = lib().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(pairs),
                               pairs.shape[0], _stream(stream))
    _check("pkv_copy_blocks", rc)


def pkv_debug_gather(k_cache: torch.Tensor, v_cache: torch.Tensor, desc: pkv_cache_desc,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, max_ctx: int,
                     k_out: torch.Tensor, v_out: torch.Tensor, stream=None) -> None:
    """k_out, v_out: [S][H_kv][max_ctx][d] in the cache dtype."""
    S = context_lens.numel()
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    _check_desc_caches(desc, k_cache, v_cache)
    need = S * desc.num_kv_heads * max_ctx * desc.head_dim * _ELEM_BYTES[desc.dtype]
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        _need(_nbytes(t) >= need, f"{name} holds {_nbytes(t)} bytes, [S][H_kv][max_ctx][d] "
                                  f"needs {need}")
    _check_device(k_cache, v_cache, block_tables, context_lens, k_out, v_out)
    rc = lib().pkv_debug_gather(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                                _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                S, max_ctx, _ptr(k_out), _ptr(v_out), _stream(stream))
    _check("pkv_debug_gather", rc)


def pkv_stream_read(buf: torch.Tensor, sink: torch.Tensor, num_workgroups: int = 0,
                    stream=None) -> None:
    """Read every byte of buf once (a streaming-read yardstick); sink: one
    int32 device word the reads are XORed into."""
    _need(sink.dtype == torch.int32 and sink.numel() >= 1, "sink must be an int32 device tensor")
    _check_device(buf, sink)
    rc = lib().pkv_stream_read(_ptr(buf), _nbytes(buf), _ptr(sink), num_workgroups,
                               _stream(stream))
    _check("pkv_stream_read", rc)


def fill_cache(k_blocks: torch.Tensor, v_blocks: torch.Tensor, desc: pkv_cache_desc,
               stream=None):
    """Cache tensors holding the given block contents.

    k_blocks, v_blocks: [num_blocks][H_kv][16][d] in the cache dtype, the token
    rows of every block in order (unused rows included). Every row is written
    with pkv_kv_append at slot block * 16 + row, the way a prefill fills a
    cache. The returned tensors have the same shape and dtype; their bytes are
    in the library's in-block layout (include/pkv.h), not in row order."""
    nb, H, B, d = k_blocks.shape
    _need(v_blocks.shape == k_blocks.shape and B == PKV_BLOCK_SIZE,
          "blocks must be [num_blocks][H_kv][16][d]")
    rows_k = k_blocks.permute(0, 2, 1, 3).reshape(nb * B, H, d).contiguous()
    rows_v = v_blocks.permute(0, 2, 1, 3).reshape(nb * B, H, d).contiguous()
    slots = torch.arange(nb * B, dtype=torch.int64, device=k_blocks.device)
    k_cache = torch.empty_like(k_blocks)
    v_cache = torch.empty_like(v_blocks)
    pkv_kv_append(rows_k, rows_v, slots, k_cache, v_cache, desc, stream)
    return k_cache, v_cache


def read_cache(k_cache: torch.Tensor, v_cache: torch.Tensor, desc: pkv_cache_desc,
               stream=None):
    """The inverse of fill_cache: the [num_blocks][H_kv][16][d] token rows of
    every block, read with pkv_debug_gather through one block table that lists
    the whole pool in order."""
    nb, H, B, d = k_cache.shape
    dev = k_cache.device
    bt = torch.arange(nb, dtype=torch.int32, device=dev).view(1, nb)
    ctx = torch.tensor([nb * B], dtype=torch.int32, device=dev)
    k_out = torch.empty((1, H, nb * B, d), dtype=k_cache.dtype, device=dev)
    v_out = torch.empty_like(k_out)
    pkv_debug_gather(k_cache, v_cache, desc, bt, ctx, nb * B, k_out, v_out, stream)
    return (k_out.view(H, nb, B, d).permute(1, 0, 2, 3).contiguous(),
            v_out.view(H, nb, B, d).permute(1, 0, 2, 3).contiguous())


# Names as the pages' problem statement gives them.
kv_append = pkv_kv_append
paged_attention_decode = pkv_paged_attention_decode
