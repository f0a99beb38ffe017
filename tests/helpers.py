"""Shared test helpers: run the HIP path through the C ABI on a DecodeBatch,
run the oracle on host copies of the same bytes, and compare.

Tolerances (written here, used by every parity test):
  * 16-bit KV (f16/bf16): max |err| <= 1e-2 and mean |err| <= 1e-3;
  * fp8 KV: max |err| <= 2e-2 (and the same mean bound, which the arithmetic
    meets: the oracle dequantises the very same codes, so only float32
    accumulation and output rounding differ);
  * float32: max |err| <= 1e-5;
  * every type also rms(err) / rms(oracle) <= 1e-2, so an output that is
    merely small (long contexts average towards 0) cannot pass by accident.
"""
import weakref

import numpy as np
import torch

import oracle
from paged_kv_cache_101_amd import binding as B
from paged_kv_cache_101_amd import workloads as W

TOL = {
    "f32": dict(max=1e-5, mean=1e-6, rel_rms=1e-5),
    "f16": dict(max=1e-2, mean=1e-3, rel_rms=1e-2),
    "bf16": dict(max=1e-2, mean=1e-3, rel_rms=1e-2),
    "fp8": dict(max=2e-2, mean=1e-3, rel_rms=1e-2),
}


def out_to_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().to(torch.float64).cpu().numpy()


def desc(b: W.DecodeBatch):
    return B.desc_for(b.k_cache, b.kv_dtype, b.k_scale, b.v_scale)


# A batch's caches (b.k_cache, b.v_cache) hold its blocks in token-row order,
# the form the oracle reads. The library's caches are built from them once
# with fill_cache (pkv_kv_append of every row) and kept per row-order tensor.
# Entries are keyed by the identity of the row-order K tensor and dropped when
# it is freed.
_DEVICE_CACHES = {}


def device_caches(b: W.DecodeBatch):
    key = id(b.k_cache)
    hit = _DEVICE_CACHES.get(key)
    if hit is None or hit[0]() is not b.k_cache or hit[1]() is not b.v_cache:
        kc, vc = B.fill_cache(b.k_cache, b.v_cache, desc(b))
        hit = (weakref.ref(b.k_cache), weakref.ref(b.v_cache), kc, vc)
        _DEVICE_CACHES[key] = hit
        weakref.finalize(b.k_cache, _DEVICE_CACHES.pop, key, None)
    return hit[2], hit[3]


def gpu_append(b: W.DecodeBatch):
    """Append the batch's new rows into its library caches (the row-order
    caches keep the state before the append)."""
    kc, vc = device_caches(b)
    B.pkv_kv_append(b.new_k, b.new_v, b.slot_mapping, kc, vc, desc(b))


def gpu_decode(b: W.DecodeBatch, num_workers=0, out=None, workspace=None,
               partition_size=0) -> torch.Tensor:
    if out is None:
        out = torch.empty_like(b.q)
    kc, vc = device_caches(b)
    B.pkv_paged_attention_decode(b.q, kc, vc, desc(b), b.block_tables, b.context_lens, b.scale,
                                 out, num_workers=num_workers, workspace=workspace,
                                 partition_size=partition_size)
    return out


def host_copy(b: W.DecodeBatch):
    return dict(q=W.to_numpy(b.q), k_cache=W.to_numpy(b.k_cache), v_cache=W.to_numpy(b.v_cache),
                bt=b.block_tables.cpu().numpy(), ctx=b.context_lens.cpu().numpy())


def oracle_decode(b: W.DecodeBatch, h=None, seqs=None) -> np.ndarray:
    """Oracle output (float64) for all sequences, or for the listed ones."""
    h = host_copy(b) if h is None else h
    q, bt, ctx = h["q"], h["bt"], h["ctx"]
    if seqs is not None:
        seqs = np.asarray(seqs)
        q, bt, ctx = (np.ascontiguousarray(q[seqs]), np.ascontiguousarray(bt[seqs]),
                      np.ascontiguousarray(ctx[seqs]))
    return oracle.paged_decode(q, h["k_cache"], h["v_cache"], bt, ctx, b.scale, b.k_scale,
                               b.v_scale)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    return dict(max=float(err.max()) if err.size else 0.0,
                mean=float(err.mean()) if err.size else 0.0,
                rel_rms=float(np.sqrt(np.mean(err ** 2)) / rms_ref) if rms_ref > 0 else 0.0,
                finite=bool(np.isfinite(got).all()))


def assert_close(got: np.ndarray, ref: np.ndarray, kv_dtype: str, what: str = ""):
    e = errors(got, ref)
    tol = TOL[kv_dtype]
    assert e["finite"], f"{what}: non-finite output"
    assert e["max"] <= tol["max"], f"{what}: max err {e['max']:.3g} > {tol['max']} ({e})"
    assert e["mean"] <= tol["mean"], f"{what}: mean err {e['mean']:.3g} > {tol['mean']} ({e})"
    assert e["rel_rms"] <= tol["rel_rms"], f"{what}: rel rms {e['rel_rms']:.3g} ({e})"
    return e


def gpu_shared_decode(b: W.DecodeBatch, num_workers=0, out=None, workspace=None,
                      group_starts=None, group_prefix=None, context_lens=None) -> torch.Tensor:
    """The shared-prefix decode of a batch, with its own prefix groups unless
    others are given."""
    if out is None:
        out = torch.empty_like(b.q)
    kc, vc = device_caches(b)
    gs = b.group_starts if group_starts is None else group_starts
    gp = b.group_prefix if group_prefix is None else group_prefix
    cl = b.context_lens if context_lens is None else context_lens
    B.pkv_paged_attention_decode_shared_prefix(b.q, kc, vc, desc(b), b.block_tables, cl, gs, gp,
                                               b.scale, out, num_workers=num_workers,
                                               workspace=workspace)
    return out
