"""Host-side checks of libpkv.so that need no GPU: it loads, exports every
entry point include/pkv.h declares, computes the sizing numbers the pages
print, and rejects every bad argument before any HIP call (so these calls
return on a machine without a GPU)."""
import ctypes
import json
import os
import re
import subprocess

import pytest
import torch

from paged_kv_cache_101_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "sizing.json")))
FAKE = 0x10000  # an aligned non-null address; never dereferenced by these calls


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(names)  # nothing else leaks out of the library


def test_sizing_matches_pages():
    g = GOLD["qwen2_5_1_5b"]
    assert B.pkv_kv_bytes_per_token(28, 2, 128, "bf16") == g["bytes_per_token"]
    g = GOLD["qwen2_5_7b"]
    assert B.pkv_kv_bytes_per_token(28, 4, 128, "bf16") == g["kib_per_token"] * 1024
    assert B.pkv_kv_bytes_per_token(28, 28, 128, "bf16") == g["mha_kib_per_token"] * 1024
    g = GOLD["gqa40_fp16"]
    assert B.pkv_kv_bytes_per_token(40, 8, 128, "f16") == g["kib_per_token"] * 1024
    assert B.pkv_kv_bytes_per_token(40, 8, 128, "fp8") == g["kib_per_token"] * 512
    assert B.pkv_kv_bytes_per_token(0, 8, 128, "f16") == 0


def test_cache_tensor_bytes():
    d = B.cache_desc(20481, 8, 128, "f16")
    assert B.pkv_cache_tensor_bytes(d) == 20481 * 8 * 16 * 128 * 2
    d = B.cache_desc(10, 8, 96, "f16")
    assert B.pkv_cache_tensor_bytes(d) == 0


def _slot_floats(gp, d):
    return gp * d + ((2 * gp + 3) // 4) * 4


def r256(x):
    return -(-x // 256) * 256


def test_workspace_bytes_formula():
    # balanced split: 2 slots per worker, then counters [S][H_kv] int32, each
    # rounded up to 256 B (max_blocks_per_seq does not enter)
    ctr = r256(40 * 8 * 4)
    ws = B.pkv_decode_workspace_bytes
    assert ws(40, 32, 8, 128, 512, 0, 2048) == r256(2 * 2048 * _slot_floats(4, 128) * 4) + ctr
    assert ws(40, 32, 8, 128, 1, 0, 0) == r256(2 * 4096 * _slot_floats(4, 128) * 4) + ctr
    # G = 6 and G = 5 use 6-head slots, G = 3 uses 4, G = 7 uses 8
    assert ws(64, 12, 2, 128, 256, 0, 10) == 512 + r256(20 * _slot_floats(6, 128) * 4)
    assert ws(1, 5, 1, 64, 1, 0, 1) == 256 + r256(2 * _slot_floats(6, 64) * 4)
    assert ws(1, 3, 1, 64, 1, 0, 1) == 256 + r256(2 * _slot_floats(4, 64) * 4)
    assert ws(1, 7, 1, 64, 1, 0, 1) == 256 + r256(2 * _slot_floats(8, 64) * 4)
    assert ws(4, 4, 3, 64, 1, 0, 1) == 0        # 4 % 3 != 0
    assert ws(4, 18, 2, 64, 1, 0, 1) == 0       # G = 9
    assert ws(4, 4, 1, 64, 1, 0, -1) == 0
    assert ws(4, 4, 1, 64, 1, 0, B.PKV_MAX_WORKERS + 1) == 0
    assert ws(4, 4, 1, 64, 0, 0, 1) == 0        # no block-table columns


def test_partition_workspace_bytes_formula():
    """Fixed partitions: one slot per (sequence, KV head, partition),
    Pn = ceil(max_blocks * 16 / P); for G = 8 (the long-context fp8 shape:
    16 x 32768, 64/8 heads, d 128, P = 512 -> Pn = 64) that is
    S * H_q * Pn * (d + 2) floats, the split-KV partial layout of
    (m_j, l_j, o_j) per (sequence, query head, partition)."""
    ws = B.pkv_decode_workspace_bytes
    S, Hq, H, d, mb = 16, 64, 8, 128, 2048
    assert ws(S, Hq, H, d, mb, 512, 0) == r256(S * Hq * 64 * (d + 2) * 4) + r256(S * H * 4)
    assert ws(S, Hq, H, d, mb, 512, 0) == 34078720 + 512
    # the worker count does not enter; a partial last partition still has a slot
    assert ws(S, Hq, H, d, mb, 512, 7) == ws(S, Hq, H, d, mb, 512, 0)
    assert ws(3, 32, 8, 128, 33, 512, 0) == r256(3 * 8 * 2 * _slot_floats(4, 128) * 4) + 256
    # P = 16: one partition per block; P past the longest context: one partition
    assert ws(2, 4, 1, 64, 5, 16, 0) == r256(2 * 1 * 5 * _slot_floats(4, 64) * 4) + 256
    assert ws(2, 4, 1, 64, 5, 4096, 0) == r256(2 * 1 * 1 * _slot_floats(4, 64) * 4) + 256
    # G = 3 pads to 4-head slots
    assert ws(2, 3, 1, 64, 4, 32, 0) == r256(2 * 1 * 2 * _slot_floats(4, 64) * 4) + 256
    for bad in (-16, 8, 520):                   # negative or not a multiple of 16
        assert ws(S, Hq, H, d, mb, bad, 0) == 0


def _decode(**kw):
    a = dict(q=FAKE, q_dtype=B.PKV_F16, S=4, Hq=8, k=FAKE, v=FAKE,
             desc=B.cache_desc(16, 2, 128, "f16"), bt=FAKE, mb=64, cl=FAKE, scale=0.1, Psz=0,
             W=0, ws=None, ws_bytes=0, out=FAKE)
    a.update(kw)
    return B.lib().pkv_paged_attention_decode(
        a["q"], a["q_dtype"], a["S"], a["Hq"], a["k"], a["v"], ctypes.byref(a["desc"]), a["bt"],
        a["mb"], a["cl"], a["scale"], a["Psz"], a["W"], a["ws"], a["ws_bytes"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.PKV_ERR_INVALID_ARG),
    (dict(out=None), B.PKV_ERR_INVALID_ARG),
    (dict(bt=None), B.PKV_ERR_INVALID_ARG),
    (dict(cl=None), B.PKV_ERR_INVALID_ARG),
    (dict(S=0), B.PKV_ERR_INVALID_ARG),
    (dict(Hq=7), B.PKV_ERR_INVALID_ARG),                      # 7 % 2 != 0
    (dict(Hq=18), B.PKV_ERR_UNSUPPORTED),                     # G = 9 > 8
    (dict(desc=B.pkv_cache_desc(16, 32, 2, 128, B.PKV_F16, 1, 1)), B.PKV_ERR_UNSUPPORTED),
    (dict(desc=B.cache_desc(16, 2, 96, "f16")), B.PKV_ERR_UNSUPPORTED),
    (dict(desc=B.cache_desc(0, 2, 128, "f16")), B.PKV_ERR_INVALID_ARG),
    (dict(q_dtype=B.PKV_BF16), B.PKV_ERR_UNSUPPORTED),        # bf16 q over f16 cache
    (dict(desc=B.cache_desc(16, 2, 128, "fp8", 0.0, 1.0), q_dtype=B.PKV_BF16),
     B.PKV_ERR_INVALID_ARG),                                  # fp8 needs positive scales
    (dict(q_dtype=7), B.PKV_ERR_UNSUPPORTED),
    (dict(W=-1), B.PKV_ERR_INVALID_ARG),                      # negative worker count
    (dict(W=B.PKV_MAX_WORKERS + 1), B.PKV_ERR_UNSUPPORTED),
    (dict(Psz=-16, ws=FAKE, ws_bytes=1 << 40), B.PKV_ERR_INVALID_ARG),  # negative partition
    (dict(Psz=24, ws=FAKE, ws_bytes=1 << 40), B.PKV_ERR_INVALID_ARG),   # not a multiple of 16
    # a balanced-split workspace is too small for 512-token partitions of this shape
    (dict(Psz=512, S=256, mb=2048, ws=FAKE, ws_bytes=B.pkv_decode_workspace_bytes(
        256, 8, 2, 128, 2048, 0, 0)), B.PKV_ERR_WORKSPACE),
    (dict(ws=None, ws_bytes=0), B.PKV_ERR_WORKSPACE),         # a workspace is always needed
    (dict(ws=FAKE, ws_bytes=100), B.PKV_ERR_WORKSPACE),
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), B.PKV_ERR_WORKSPACE),  # not 256-byte aligned
    (dict(q=FAKE + 4), B.PKV_ERR_INVALID_ARG),                # misaligned
    (dict(scale=float("nan")), B.PKV_ERR_INVALID_ARG),
])
def test_decode_rejects_before_any_hip_call(kw, status):
    assert _decode(**kw) == status


def _append(**kw):
    a = dict(k=FAKE, v=FAKE, dt=B.PKV_F16, slots=FAKE, T=4, kc=FAKE, vc=FAKE,
             desc=B.cache_desc(16, 2, 128, "f16"))
    a.update(kw)
    return B.lib().pkv_kv_append(a["k"], a["v"], a["dt"], a["slots"], a["T"], a["kc"], a["vc"],
                                 ctypes.byref(a["desc"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), B.PKV_ERR_INVALID_ARG),
    (dict(slots=None), B.PKV_ERR_INVALID_ARG),
    (dict(kc=None), B.PKV_ERR_INVALID_ARG),
    (dict(T=-1), B.PKV_ERR_INVALID_ARG),
    (dict(dt=B.PKV_BF16), B.PKV_ERR_UNSUPPORTED),             # not the cache dtype
    (dict(desc=B.pkv_cache_desc(16, 8, 2, 128, B.PKV_F16, 1, 1)), B.PKV_ERR_UNSUPPORTED),
    (dict(v=FAKE + 8), B.PKV_ERR_INVALID_ARG),
    (dict(T=0, k=None, v=None, slots=None), B.PKV_OK),        # empty append is a no-op
    # quantising append: 16/32-bit rows into an fp8 cache, never the reverse
    (dict(T=0, dt=B.PKV_BF16, desc=B.cache_desc(16, 2, 128, "fp8", 0.5, 0.5)), B.PKV_OK),
    (dict(T=0, dt=B.PKV_F32, desc=B.cache_desc(16, 2, 128, "fp8", 0.5, 0.5)), B.PKV_OK),
    (dict(dt=B.PKV_FP8_E4M3), B.PKV_ERR_UNSUPPORTED),         # fp8 rows into an f16 cache
    (dict(dt=B.PKV_F16, desc=B.cache_desc(16, 2, 128, "fp8", 0.0, 0.5)), B.PKV_ERR_INVALID_ARG),
])
def test_append_rejects_before_any_hip_call(kw, status):
    assert _append(**kw) == status


def test_shared_prefix_workspace_bytes_formula():
    S, Hq, H, d, ng, W = 256, 32, 8, 128, 3, 768
    base = B.pkv_decode_workspace_bytes(S, Hq, H, d, 1, 0, W)  # decode slots + counters
    res = r256(S * Hq * d * 4) + r256(S * Hq * 4)
    slots = r256(4096 * (16 * d + 32) * 4)
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, ng, W) == base + res + slots
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, ng, 0) == \
        B.pkv_decode_workspace_bytes(S, Hq, H, d, 1, 0, 0) + res + slots
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, -1, W) == 0
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, S + 1, W) == 0
    assert B.pkv_shared_prefix_workspace_bytes(4, 18, 2, 64, 1, 1) == 0  # G = 9


def _shared(**kw):
    a = dict(q=FAKE, q_dtype=B.PKV_BF16, S=4, Hq=8, k=FAKE, v=FAKE,
             desc=B.cache_desc(16, 2, 128, "bf16"), bt=FAKE, mb=64, cl=FAKE, ng=1, gs=FAKE,
             gp=FAKE, scale=0.1, P=0, ws=FAKE, ws_bytes=1 << 40, out=FAKE)
    a.update(kw)
    return B.lib().pkv_paged_attention_decode_shared_prefix(
        a["q"], a["q_dtype"], a["S"], a["Hq"], a["k"], a["v"], ctypes.byref(a["desc"]), a["bt"],
        a["mb"], a["cl"], a["ng"], a["gs"], a["gp"], a["scale"], a["P"], a["ws"], a["ws_bytes"],
        a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ng=-1), B.PKV_ERR_INVALID_ARG),
    (dict(ng=5), B.PKV_ERR_INVALID_ARG),                      # more groups than sequences
    (dict(gs=None), B.PKV_ERR_INVALID_ARG),
    (dict(gp=None), B.PKV_ERR_INVALID_ARG),
    (dict(q=None), B.PKV_ERR_INVALID_ARG),
    (dict(Hq=18), B.PKV_ERR_UNSUPPORTED),
    (dict(q_dtype=B.PKV_F16), B.PKV_ERR_UNSUPPORTED),         # f16 q over a bf16 cache
    (dict(ws=None), B.PKV_ERR_WORKSPACE),
    (dict(ws_bytes=1 << 20), B.PKV_ERR_WORKSPACE),            # a decode-sized one is too small
    (dict(ws=FAKE + 16), B.PKV_ERR_WORKSPACE),
])
def test_shared_prefix_rejects_before_any_hip_call(kw, status):
    assert _shared(**kw) == status


def test_prefill_workspace_bytes_formula():
    for d in (64, 128):
        assert B.pkv_prefill_workspace_bytes(d) == r256(4096 * (16 * d + 32) * 4)
    assert B.pkv_prefill_workspace_bytes(96) == 0


def _prefill(**kw):
    a = dict(q=FAKE, q_dtype=B.PKV_F16, S=2, T=10, Hq=8, qs=FAKE, k=FAKE, v=FAKE,
             desc=B.cache_desc(16, 2, 128, "f16"), bt=FAKE, mb=64, cl=FAKE, scale=0.1,
             ws=None, ws_bytes=0, out=FAKE)
    a.update(kw)
    return B.lib().pkv_paged_attention_prefill(
        a["q"], a["q_dtype"], a["S"], a["T"], a["Hq"], a["qs"], a["k"], a["v"],
        ctypes.byref(a["desc"]), a["bt"], a["mb"], a["cl"], a["scale"], a["ws"], a["ws_bytes"],
        a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), B.PKV_ERR_INVALID_ARG),
    (dict(qs=None), B.PKV_ERR_INVALID_ARG),
    (dict(T=0, q=None, out=None), B.PKV_OK),                  # nothing to compute
    (dict(q=None), B.PKV_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), B.PKV_ERR_INVALID_ARG),              # misaligned
    (dict(Hq=7), B.PKV_ERR_INVALID_ARG),
    (dict(Hq=18), B.PKV_ERR_UNSUPPORTED),                     # G = 9
    (dict(q_dtype=B.PKV_BF16), B.PKV_ERR_UNSUPPORTED),        # bf16 q over an f16 cache
    (dict(desc=B.cache_desc(16, 2, 96, "f16")), B.PKV_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), B.PKV_ERR_INVALID_ARG),
    (dict(ws=FAKE, ws_bytes=1 << 20), B.PKV_ERR_WORKSPACE),   # too small for the slots
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), B.PKV_ERR_WORKSPACE),  # not 256-byte aligned
])
def test_prefill_rejects_before_any_hip_call(kw, status):
    assert _prefill(**kw) == status


def test_copy_blocks_rejects_bad_args():
    L = B.lib()
    d = B.cache_desc(16, 2, 128, "f16")
    assert L.pkv_copy_blocks(FAKE, FAKE, ctypes.byref(d), None, 3, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_copy_blocks(FAKE, FAKE, ctypes.byref(d), FAKE, -1, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_copy_blocks(None, FAKE, ctypes.byref(d), FAKE, 1, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_copy_blocks(FAKE + 8, FAKE, ctypes.byref(d), FAKE, 1, None) == B.PKV_ERR_INVALID_ARG
    bad = B.cache_desc(16, 2, 96, "f16")
    assert L.pkv_copy_blocks(FAKE, FAKE, ctypes.byref(bad), FAKE, 1, None) == B.PKV_ERR_UNSUPPORTED
    assert L.pkv_copy_blocks(FAKE, FAKE, ctypes.byref(d), None, 0, None) == B.PKV_OK  # nothing to do


def test_gather_rejects_bad_args():
    L = B.lib()
    d = B.cache_desc(16, 2, 128, "f16")
    assert L.pkv_debug_gather(FAKE, FAKE, ctypes.byref(d), FAKE, 4, FAKE, 0, 8, FAKE, FAKE,
                              None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_debug_gather(FAKE, FAKE, ctypes.byref(d), None, 4, FAKE, 2, 8, FAKE, FAKE,
                              None) == B.PKV_ERR_INVALID_ARG


def test_noalloc_rejects_before_any_hip_call():
    """The allocation-free decode checks its arguments like decode, and a
    batch whose workspace would exceed the static scratch is refused before
    any HIP call."""
    L = B.lib()

    def call(S=4, Hq=8, mb=64, P=0, W=0, q=FAKE):
        return L.pkv_paged_attention_decode_noalloc(
            q, B.PKV_F16, S, Hq, FAKE, FAKE, ctypes.byref(B.cache_desc(16, 2, 128, "f16")), FAKE,
            mb, FAKE, 0.1, P, W, FAKE, None)
    assert call(q=None) == B.PKV_ERR_INVALID_ARG
    assert call(Hq=18) == B.PKV_ERR_UNSUPPORTED
    assert call(P=24) == B.PKV_ERR_INVALID_ARG
    assert call(W=-1) == B.PKV_ERR_INVALID_ARG
    # 256 sequences x 2 KV heads x 2048 blocks in 16-token partitions: far past the scratch
    assert B.pkv_decode_workspace_bytes(256, 8, 2, 128, 2048, 16, 0) > B.PKV_NOALLOC_SCRATCH_BYTES
    assert call(S=256, mb=2048, P=16) == B.PKV_ERR_TOO_LARGE
    # the long-context fp8 shape at 512-token partitions fits
    assert B.pkv_decode_workspace_bytes(16, 64, 8, 128, 2048, 512, 0) <= B.PKV_NOALLOC_SCRATCH_BYTES
    # so does the default worker count at the largest group and head size
    assert B.pkv_decode_workspace_bytes(1024, 64, 8, 128, 1, 0, 0) <= B.PKV_NOALLOC_SCRATCH_BYTES


def test_stream_read_rejects_bad_args():
    L = B.lib()
    assert L.pkv_stream_read(None, 16, FAKE, 0, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read(FAKE, 16, None, 0, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read(FAKE + 8, 16, FAKE, 0, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read(FAKE, 20, FAKE, 0, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read(FAKE, 16, FAKE, -1, None) == B.PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read(FAKE, 0, FAKE, 0, None) == B.PKV_OK


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 99):
        assert B.status_string(s)


# ---- the Python binding checks tensors against the descriptor -----------------
# (the C side sees pointers only; these checks run before any library call,
# so CPU tensors show them)

def _decode_tensors(S=4, Hq=8, H=2, d=128, nb=16, mb=4, dt=torch.float16):
    q = torch.zeros((S, Hq, d), dtype=dt)
    kc = torch.zeros((nb, H, 16, d), dtype=dt)
    return dict(q=q, k_cache=kc, v_cache=kc.clone(), block_tables=torch.zeros((S, mb), dtype=torch.int32),
                context_lens=torch.ones(S, dtype=torch.int32), out=torch.empty_like(q))


@pytest.mark.parametrize("change,msg", [
    (dict(desc=B.cache_desc(16, 2, 64, "f16")), "head_dim"),          # q's d != desc's
    (dict(desc=B.cache_desc(16, 3, 128, "f16")), "multiple of num_kv_heads"),
    (dict(desc=B.cache_desc(17, 2, 128, "f16")), "pool needs"),       # caches too small
    (dict(desc=B.cache_desc(16, 2, 128, "bf16")), "does not match"),  # cache dtype
    (dict(out=torch.zeros((4, 8, 64), dtype=torch.float16)), "out must match q"),
    (dict(block_tables=torch.zeros((3, 4), dtype=torch.int32)), "block_tables"),
    (dict(context_lens=torch.ones(4, dtype=torch.int64)), "context_lens"),
])
def test_binding_decode_rejects_mismatch(change, msg):
    t = _decode_tensors()
    desc = change.pop("desc", B.cache_desc(16, 2, 128, "f16"))
    t.update(change)
    with pytest.raises(ValueError, match=msg):
        B.pkv_paged_attention_decode(t["q"], t["k_cache"], t["v_cache"], desc, t["block_tables"],
                                     t["context_lens"], 0.1, t["out"])
    with pytest.raises(ValueError, match=msg):
        B.pkv_paged_attention_decode_shared_prefix(
            t["q"], t["k_cache"], t["v_cache"], desc, t["block_tables"], t["context_lens"],
            torch.tensor([0, 4], dtype=torch.int32), torch.tensor([1], dtype=torch.int32), 0.1,
            t["out"])


def test_binding_decode_checks_device_last():
    """Matching CPU tensors pass every shape check and stop at the device check."""
    t = _decode_tensors()
    with pytest.raises(ValueError, match="device tensors"):
        B.pkv_paged_attention_decode(t["q"], t["k_cache"], t["v_cache"],
                                     B.cache_desc(16, 2, 128, "f16"), t["block_tables"],
                                     t["context_lens"], 0.1, t["out"])


def test_binding_prefill_rejects_mismatch():
    t = _decode_tensors()
    qs = torch.tensor([0, 1, 2, 3, 4], dtype=torch.int32)
    for desc, msg in ((B.cache_desc(16, 2, 64, "f16"), "head_dim"),
                      (B.cache_desc(32, 2, 128, "f16"), "pool needs")):
        with pytest.raises(ValueError, match=msg):
            B.pkv_paged_attention_prefill(t["q"], t["k_cache"], t["v_cache"], desc,
                                          t["block_tables"], t["context_lens"], qs, 0.1, t["out"])


def test_binding_append_rejects_mismatch():
    kc = torch.zeros((16, 2, 16, 128), dtype=torch.float16)
    k = torch.zeros((3, 2, 128), dtype=torch.float16)
    slots = torch.zeros(3, dtype=torch.int64)
    for desc, kk, msg in ((B.cache_desc(16, 4, 128, "f16"), k, "heads"),
                          (B.cache_desc(16, 2, 64, "f16"), k, "head_dim"),
                          (B.cache_desc(20, 2, 128, "f16"), k, "pool needs"),
                          (B.cache_desc(16, 2, 128, "f16"), torch.zeros((3, 2, 64), dtype=torch.float16),
                           "head_dim")):
        with pytest.raises(ValueError, match=msg):
            B.pkv_kv_append(kk, kk.clone(), slots, kc, kc.clone(), desc)


def test_binding_gather_and_copy_reject_mismatch():
    kc = torch.zeros((16, 2, 16, 64), dtype=torch.float32)
    desc = B.cache_desc(16, 2, 64, "f32")
    bt = torch.zeros((2, 3), dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    small = torch.zeros((2, 2, 40, 64), dtype=torch.float32)   # max_ctx 48 needs 48 rows
    with pytest.raises(ValueError, match="k_out"):
        B.pkv_debug_gather(kc, kc.clone(), desc, bt, cl, 48, small, small.clone())
    with pytest.raises(ValueError, match="pool needs"):
        B.pkv_copy_blocks(kc, kc.clone(), B.cache_desc(32, 2, 64, "f32"),
                          torch.zeros((1, 2), dtype=torch.int32))


C_CALLER = r"""
#include "pkv.h"
#include "pkv_blocks.h"
#include <stdio.h>

int main(void) {
    /* sizing and the block manager run on the host */
    size_t ws = pkv_decode_workspace_bytes(40, 32, 8, 128, 512, 0, 0);
    size_t kv = pkv_kv_bytes_per_token(40, 8, 128, PKV_F16);
    pkv_block_manager *bm = pkv_bm_create(64, 1);
    if (bm == NULL) return 2;
    int64_t prompt[20];
    for (int i = 0; i < 20; ++i) prompt[i] = 100 + i;
    int32_t cached = -1, ncopies = -1, copies[1][2];
    int64_t slots[20];
    int rc = pkv_bm_add_request(bm, 7, prompt, 20, 0, &cached);
    rc |= pkv_bm_append(bm, 7, 20, NULL, slots, copies, &ncopies);
    int32_t nblocks = pkv_bm_num_blocks(bm, 7), free_blocks = pkv_bm_num_free_blocks(bm);
    pkv_bm_destroy(bm);
    printf("%zu %zu %d %d %d %d %d\n", ws, kv, rc, cached, ncopies, nblocks, free_blocks);
    return 0;
}
"""


def test_headers_serve_a_plain_c_caller(tmp_path):
    """include/pkv.h and include/pkv_blocks.h compile as strict C99 (no HIP
    header needed), and a C program links libpkv.so and calls its host
    entry points."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    B.lib()  # raises if the library has not been built
    src, exe = tmp_path / "caller.c", tmp_path / "caller"
    src.write_text(C_CALLER)
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{os.path.join(ROOT, 'include')}", str(src), f"-L{libdir}", "-lpkv",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    ws, kv, rc, cached, ncopies, nblocks, free_blocks = map(int, out)
    assert ws == B.pkv_decode_workspace_bytes(40, 32, 8, 128, 512, 0, 0)
    assert kv == 40 * 2 * 8 * 128 * 2  # the pages' per-token formula, 40 layers, fp16
    assert (rc, cached, ncopies, nblocks) == (0, 0, 0, 2)
    assert free_blocks == 63 - 2
