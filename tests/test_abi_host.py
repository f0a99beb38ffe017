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
    # 2 slots per worker, then counters [S][H_kv] int32, each rounded up to 256 B
    ctr = r256(40 * 8 * 4)
    assert B.pkv_decode_workspace_bytes(40, 32, 8, 128, 2048) == r256(2 * 2048 * _slot_floats(4, 128) * 4) + ctr
    assert B.pkv_decode_workspace_bytes(40, 32, 8, 128, 0) == r256(2 * 4096 * _slot_floats(4, 128) * 4) + ctr
    # G = 6 and G = 5 use 6-head slots, G = 3 uses 4, G = 7 uses 8
    assert B.pkv_decode_workspace_bytes(64, 12, 2, 128, 10) == 512 + r256(20 * _slot_floats(6, 128) * 4)
    assert B.pkv_decode_workspace_bytes(1, 5, 1, 64, 1) == 256 + r256(2 * _slot_floats(6, 64) * 4)
    assert B.pkv_decode_workspace_bytes(1, 3, 1, 64, 1) == 256 + r256(2 * _slot_floats(4, 64) * 4)
    assert B.pkv_decode_workspace_bytes(1, 7, 1, 64, 1) == 256 + r256(2 * _slot_floats(8, 64) * 4)
    assert B.pkv_decode_workspace_bytes(4, 4, 3, 64, 1) == 0        # 4 % 3 != 0
    assert B.pkv_decode_workspace_bytes(4, 18, 2, 64, 1) == 0       # G = 9
    assert B.pkv_decode_workspace_bytes(4, 4, 1, 64, -1) == 0
    assert B.pkv_decode_workspace_bytes(4, 4, 1, 64, B.PKV_MAX_WORKERS + 1) == 0


def _decode(**kw):
    a = dict(q=FAKE, q_dtype=B.PKV_F16, S=4, Hq=8, k=FAKE, v=FAKE,
             desc=B.cache_desc(16, 2, 128, "f16"), bt=FAKE, mb=64, cl=FAKE, scale=0.1, P=0,
             ws=None, ws_bytes=0, out=FAKE)
    a.update(kw)
    return B.lib().pkv_paged_attention_decode(
        a["q"], a["q_dtype"], a["S"], a["Hq"], a["k"], a["v"], ctypes.byref(a["desc"]), a["bt"],
        a["mb"], a["cl"], a["scale"], a["P"], a["ws"], a["ws_bytes"], a["out"], None)


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
    (dict(P=-1), B.PKV_ERR_INVALID_ARG),                      # negative worker count
    (dict(P=B.PKV_MAX_WORKERS + 1), B.PKV_ERR_UNSUPPORTED),
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
    base = B.pkv_decode_workspace_bytes(S, Hq, H, d, W)  # decode slots + decode counters
    res = r256(S * Hq * d * 4) + r256(S * Hq * 4)
    slots = r256(4096 * (16 * d + 32) * 4)
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, ng, W) == base + res + slots
    assert B.pkv_shared_prefix_workspace_bytes(S, Hq, H, d, ng, 0) == \
        B.pkv_decode_workspace_bytes(S, Hq, H, d, 0) + res + slots
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


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 99):
        assert B.status_string(s)
