"""GPU: the allocation-free decode entry point against the decode entry point.

pkv_paged_attention_decode_noalloc runs the same kernels as
pkv_paged_attention_decode with the library's static per-GPU scratch as the
workspace. For the same arguments (worker count, partition size) its output
must equal the workspace call's bit for bit, and both must match the oracle
within the tolerances of the parity tests. Two calls in a row, the second on
a smaller batch, check that the scratch left by one call does not leak into
the next."""
import numpy as np
import pytest
import torch

from paged_kv_cache_101_amd import binding as B
from paged_kv_cache_101_amd import workloads as W
from tests.helpers import assert_close, desc, device_caches, gpu_decode, oracle_decode, out_to_f64

pytestmark = pytest.mark.gpu


def _noalloc(b, num_workers=0, partition_size=0):
    out = torch.empty_like(b.q)
    kc, vc = device_caches(b)
    B.pkv_paged_attention_decode_noalloc(b.q, kc, vc, desc(b), b.block_tables, b.context_lens,
                                         b.scale, out, num_workers=num_workers,
                                         partition_size=partition_size)
    return out


@pytest.mark.parametrize("nw,P", [(0, 0), (37, 0), (0, 512), (5, 64)])
def test_noalloc_matches_decode_two_calls(gpu, nw, P):
    big = W.make_batch("noalloc-big", 91, [3000, 17, 4500, 900, 1, 2500, 8192], 32, 8, 128, "f16",
                       "f16", device=gpu, canary=True)
    small = W.make_batch("noalloc-small", 92, [700, 33], 32, 8, 128, "f16", "f16", device=gpu,
                         canary=True)
    for b in (big, small):  # the second call is on a smaller batch
        print(f"[case] noalloc S={b.num_seqs} workers={nw} partition={P}", flush=True)
        got = _noalloc(b, nw, P)
        want = gpu_decode(b, nw, partition_size=P)
        torch.cuda.synchronize()
        assert W.to_numpy(got).tobytes() == W.to_numpy(want).tobytes(), \
            f"S={b.num_seqs}: noalloc differs from the workspace call"
        e = assert_close(out_to_f64(got), oracle_decode(b), "f16", f"noalloc S={b.num_seqs}")
        print(f"[parity] noalloc S={b.num_seqs} workers={nw} P={P}: {e}", flush=True)


def test_noalloc_long_context_fp8_sampled(gpu):
    """The long-context fp8 workload at full size with 512-token partitions
    (the largest shape the scratch is sized for), then a small bf16 batch."""
    b = W.fp8_long(device=gpu)
    got = _noalloc(b, partition_size=512)
    want = gpu_decode(b, partition_size=512)
    torch.cuda.synchronize()
    assert W.to_numpy(got).tobytes() == W.to_numpy(want).tobytes()
    seqs = [3, 12]
    assert_close(out_to_f64(got)[np.asarray(seqs)], oracle_decode(b, seqs=seqs), "fp8", "noalloc fp8")
    s = W.make_batch("noalloc-after", 93, [40, 1, 300], 12, 2, 128, "bf16", "bf16", device=gpu,
                     canary=True)
    got = _noalloc(s)
    torch.cuda.synchronize()
    assert_close(out_to_f64(got), oracle_decode(s), "bf16", "noalloc after fp8")


def test_noalloc_too_large_is_refused(gpu):
    b = W.make_batch("noalloc-refuse", 94, [16] * 4, 8, 2, 128, "f16", "f16", device=gpu)
    kc, vc = device_caches(b)
    big_bt = torch.zeros((4, 1 << 20), dtype=torch.int32, device=gpu)  # 16M-token rows
    with pytest.raises(B.PkvError) as ei:
        B.pkv_paged_attention_decode_noalloc(b.q, kc, vc, desc(b), big_bt, b.context_lens, b.scale,
                                             torch.empty_like(b.q), partition_size=16)
    assert ei.value.status == B.PKV_ERR_TOO_LARGE
