"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libpkv.so (hand-written HIP kernels behind the C ABI
of include/pkv.h); ``binding`` is its ctypes wrapper and ``workloads`` builds
seeded synthetic inputs. Importing the package loads nothing: the library is
opened on first use and a missing library raises.
"""
from .binding import (  # noqa: F401
    PkvError,
    cache_desc,
    decode_workspace,
    desc_for,
    kv_append,
    paged_attention_decode,
    pkv_cache_tensor_bytes,
    pkv_debug_gather,
    pkv_decode_workspace_bytes,
    pkv_kv_append,
    pkv_kv_bytes_per_token,
    pkv_paged_attention_decode,
)
