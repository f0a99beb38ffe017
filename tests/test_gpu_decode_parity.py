"""GPU: paged decode attention against the oracle, element by element.

Reduced sizes run the whole batch through the oracle; the full-size
workloads run in the launch configuration the benchmark times (the device
default worker count) and the oracle recomputes every sequence (a few
seconds of double-precision work on the host cores per workload). Forced worker counts exercise other split-KV patterns: a single worker
(no split at all), a few (every segment split at odd places), and more
workers than tiles."""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_101_amd import workloads as W
from tests.helpers import (assert_close, gpu_append, gpu_decode, host_copy, oracle_decode,
                           out_to_f64)

pytestmark = pytest.mark.gpu


def _check(b, num_workers=0, seqs=None, what="", partition_size=0):
    out = gpu_decode(b, num_workers, partition_size=partition_size)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    ref = oracle_decode(b, seqs=seqs)
    if seqs is not None:
        got = got[np.asarray(seqs)]
    e = assert_close(got, ref, b.kv_dtype, what or b.name)
    print(f"[parity] {what or b.name}: {e}", flush=True)
    return got, ref


def test_tiny(gpu):
    _check(W.tiny(device=gpu, canary=True))


@pytest.mark.parametrize("nw", [1, 2, 3, 5, 6, 64])
def test_tiny_workers(gpu, nw):
    _check(W.tiny(device=gpu, canary=True), num_workers=nw, what=f"tiny workers={nw}")


def test_qwen_layer_append_then_decode(gpu):
    """The full Qwen2.5-1.5B-shaped layer: append one token per sequence (its
    slot held NaN before), then decode; the oracle does the same on the host."""
    b = W.qwen_layer(device=gpu, canary=True)
    h = host_copy(b)
    gpu_append(b)
    out = gpu_decode(b)
    torch.cuda.synchronize()
    oracle.kv_append(W.to_numpy(b.new_k), W.to_numpy(b.new_v), b.slot_mapping.cpu().numpy(),
                     h["k_cache"], h["v_cache"])
    ref = oracle.paged_decode(h["q"], h["k_cache"], h["v_cache"], h["bt"], h["ctx"], b.scale)
    e = assert_close(out_to_f64(out), ref, "bf16", "qwen layer")
    print(f"[parity] qwen layer append+decode: {e}", flush=True)


def test_gqa40_reduced(gpu):
    _check(W.gqa40_layer(device=gpu, num_seqs=6, ctx=8192, canary=True), what="gqa40 6x8192")


def test_gqa40_ragged_lengths(gpu):
    ctx = [1, 15, 16, 17, 511, 512, 513, 1000, 4097, 8192]
    b = W.make_batch("gqa40-ragged", 31, ctx, 32, 8, 128, "f16", "f16", device=gpu, canary=True)
    for nw in (0, 1, 7, 64, 333, 4096):
        _check(b, num_workers=nw, what=f"gqa40 ragged workers={nw}")


def test_gqa40_full_layer(gpu):
    """One layer of the 40-layer workload at full size (40 x 8192, 32/8 heads,
    fp16, 20,481-block pool), device-default workers, as the benchmark times
    it; the oracle recomputes every sequence (about 2.7 G multiply-adds in
    double precision, a few seconds on the host cores)."""
    _check(W.gqa40_layer(device=gpu, layer=3), what="gqa40 full")


def test_gqa40_tp8_share(gpu):
    """One GPU's share of the 40-layer workload under 8-way KV-head
    parallelism (40 x 8192, 4 query / 1 KV head, fp16), the bench's gqa40_tp8
    layer at full size; the oracle recomputes every sequence."""
    _check(W.gqa40_tp8_layer(device=gpu, layer=5, canary=True), what="gqa40 tp8 share")


def test_prefix_shared_reduced(gpu):
    _check(W.prefix_shared(device=gpu, num_seqs=24, canary=True), what="prefix 24 seqs")


def test_prefix_shared_full(gpu):
    """The prefix-sharing workload at full size (256 sequences, a 2048-token
    shared prefix plus 64..512-token suffixes) through plain decode; the
    oracle recomputes every sequence."""
    _check(W.prefix_shared(device=gpu), what="prefix full")


def test_fp8_reduced(gpu):
    b = W.make_batch("fp8-reduced", 51, [1, 100, 511, 513, 4000], 64, 8, 128, "fp8", "bf16",
                     device=gpu, canary=True)
    _check(b, what="fp8 ragged")


def test_fp8_f16_query(gpu):
    b = W.make_batch("fp8-f16q", 52, [33, 700, 1500], 16, 2, 128, "fp8", "f16", device=gpu,
                     canary=True)
    _check(b, what="fp8 f16 q")


def test_fp8_full(gpu):
    """The long-context fp8 workload at full size (16 x 32768, 64/8 heads),
    balanced split; the oracle recomputes every sequence."""
    _check(W.fp8_long(device=gpu), what="fp8 full")


def test_fp8_full_partition_512(gpu):
    """The long-context fp8 workload at full size split into 512-token
    partitions (64 per sequence, merged by log-sum-exp), the device-default
    worker count for that split; the oracle recomputes every sequence. The
    balanced split of the same batch agrees to float32 rounding."""
    b = W.fp8_long(device=gpu)
    got, ref = _check(b, partition_size=512, what="fp8 full P=512")
    bal = out_to_f64(gpu_decode(b))
    assert np.abs(bal - got).max() <= 2e-2


@pytest.mark.parametrize("P", [16, 48, 512, 8192, 16384])
def test_fixed_partitions_ragged(gpu, P):
    """Fixed partitions of P tokens over ragged lengths (one partition, a
    partial last partition, up to 512 partitions per segment), several
    worker counts (each wave holding whole partitions)."""
    ctx = [1, 15, 16, 17, 511, 512, 513, 1000, 4097, 8192]
    b = W.make_batch("gqa40-ragged", 31, ctx, 32, 8, 128, "f16", "f16", device=gpu, canary=True)
    for nw in (0, 1, 7, 333, 4096):
        _check(b, num_workers=nw, partition_size=P, what=f"ragged P={P} workers={nw}")


@pytest.mark.parametrize("Hq,H,d,kv", [(4, 1, 64, "f32"), (6, 2, 64, "bf16"), (7, 1, 128, "f16"),
                                       (16, 2, 64, "fp8"), (8, 1, 128, "bf16")])
def test_fixed_partitions_head_shapes(gpu, Hq, H, d, kv):
    q_dtype = "bf16" if kv == "fp8" else kv
    b = W.make_batch("shapes-part", 161 + Hq + H, [1, 5, 16, 47, 300, 1100, 2049], Hq, H, d, kv,
                     q_dtype, device=gpu, canary=True)
    for P, nw in ((32, 0), (64, 3), (256, 50)):
        _check(b, num_workers=nw, partition_size=P,
               what=f"Hq={Hq} H={H} d={d} {kv} P={P} workers={nw}")


@pytest.mark.parametrize("Hq,H,d,kv", [(4, 1, 64, "f32"), (8, 8, 64, "f16"), (6, 2, 64, "bf16"),
                                       (7, 1, 128, "f16"), (3, 3, 128, "bf16"), (10, 2, 64, "fp8"),
                                       (5, 5, 128, "f32"), (16, 2, 64, "f16")])
def test_head_shapes(gpu, Hq, H, d, kv):
    q_dtype = "bf16" if kv == "fp8" else kv
    b = W.make_batch("shapes", 61 + Hq + H, [1, 5, 16, 47, 300, 1100], Hq, H, d, kv, q_dtype,
                     device=gpu, canary=True)
    for nw in (0, 3, 50):
        _check(b, num_workers=nw, what=f"Hq={Hq} H={H} d={d} {kv} workers={nw}")


def test_empty_and_zero_lengths(gpu):
    b = W.make_batch("empty", 71, [0, 3, 0, 40], 8, 2, 128, "bf16", "bf16", device=gpu,
                     canary=True, max_blocks=40)
    for nw in (0, 1, 4):
        got, _ = _check(b, num_workers=nw, what=f"zero lengths workers={nw}")
        assert (got[0] == 0).all() and (got[2] == 0).all()


def test_invalid_metadata_gives_nan_rows_not_faults(gpu):
    b = W.make_batch("bad", 72, [40, 40, 40], 4, 1, 64, "f16", "f16", device=gpu, max_blocks=4)
    bt = b.block_tables.clone()
    bt[1, 1] = b.num_blocks + 5     # block id past the pool
    bt[2, 0] = -3                   # negative block id
    b.block_tables = bt
    cl = b.context_lens.clone()
    cl[0] = 4 * 16 + 1              # longer than the block table row
    for nw in (0, 1, 5):
        out = gpu_decode(W.DecodeBatch(**{**b.__dict__, "context_lens": cl}), nw)
        torch.cuda.synchronize()
        o = out_to_f64(out)
        assert np.isnan(o).all(), f"workers={nw}"


def test_one_long_sequence_many_partials(gpu):
    """One sequence, one KV head: every worker holds a slice of the same
    segment, and the last one merges them all (up to 2048 partials)."""
    b = W.make_batch("one-long", 73, [32768], 8, 1, 128, "bf16", "bf16", device=gpu, canary=True)
    for nw in (0, 2, 100, 2048):
        _check(b, num_workers=nw, what=f"1 x 32768 workers={nw}")


def test_workspace_reuse_leaves_counters_zero(gpu):
    """Back-to-back calls on one workspace (the counters must come back to
    zero after every call) give identical bytes, and the counters are zero."""
    from paged_kv_cache_101_amd import binding as B
    b = W.make_batch("reuse", 74, [3000, 17, 4500, 900], 32, 8, 128, "f16", "f16", device=gpu)
    ws = B.decode_workspace(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, 37, gpu)
    first = gpu_decode(b, 37, workspace=ws)
    for _ in range(4):
        again = gpu_decode(b, 37, workspace=ws)
        assert W.to_numpy(again).tobytes() == W.to_numpy(first).tobytes()
    torch.cuda.synchronize()
    # the counters [S][H_kv] sit in the workspace's last 256-byte-rounded bytes
    assert int(ws[-256:].view(torch.int32).abs().sum()) == 0
    ref = oracle_decode(b)
    assert_close(out_to_f64(first), ref, "f16", "reuse")


def test_workspace_sized_once_serves_smaller_calls(gpu):
    """A workspace sized for the largest shape and zeroed once serves calls
    with fewer sequences and other worker counts, in any order."""
    from paged_kv_cache_101_amd import binding as B
    big = W.make_batch("ws-big", 75, [3000, 17, 4500, 900, 64, 2500], 32, 8, 128, "f16", "f16",
                       device=gpu)
    small = W.make_batch("ws-small", 76, [700, 5000], 32, 8, 128, "f16", "f16", device=gpu)
    ws = B.decode_workspace(6, 32, 8, 128, 0, gpu)
    ref_big, ref_small = oracle_decode(big), oracle_decode(small)
    for b, nw, ref in ((small, 0, ref_small), (big, 300, ref_big), (small, 5, ref_small),
                       (big, 0, ref_big), (small, 2048, ref_small), (big, 1, ref_big)):
        got = gpu_decode(b, nw, workspace=ws)
        assert_close(out_to_f64(got), ref, "f16", f"S={b.num_seqs} workers={nw}")
