"""GPU: decode and the shared-prefix decode on seeded random batches against
the oracle.

Each case draws its own shape: the cache type (and the query type that goes
with it), d 64 or 128, G = 1..8, 1..4 KV heads, and ragged context lengths
from one token to a few thousand (short, medium and long ones mixed), with the
device's default worker count or a random one, and the balanced split or
fixed partitions of a random size. The shared-prefix cases also
draw contiguous prefix groups (0..20 shared blocks, members holding their
prefix plus 0..100 tokens) with ungrouped sequences between them."""
import numpy as np
import pytest

from paged_kv_cache_101_amd import workloads as W
from tests.helpers import assert_close, gpu_decode, gpu_shared_decode, oracle_decode, out_to_f64

pytestmark = pytest.mark.gpu

BLOCK = 16
TYPES = [("bf16", "bf16"), ("f16", "f16"), ("fp8", "bf16"), ("fp8", "f16"), ("f32", "f32")]


def _heads(rng, d):
    G = int(rng.integers(1, 9))
    H = int(rng.integers(1, 5))
    return G * H, H


def _length(rng):
    u = rng.random()
    if u < 0.3:
        return int(rng.integers(1, 65))
    if u < 0.8:
        return int(rng.integers(65, 2001))
    return int(rng.integers(2001, 6001))


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(gpu, seed):
    rng = np.random.default_rng(7000 + seed)
    kv, qd = TYPES[seed % len(TYPES)]
    d = (64, 128)[int(rng.integers(0, 2))]
    Hq, H = _heads(rng, d)
    S = int(rng.integers(1, 49))
    ctx = [_length(rng) for _ in range(S)]
    workers = 0 if rng.random() < 0.5 else int(rng.integers(1, 301))
    # the balanced split, or fixed partitions of 16..1024 tokens
    part = 0 if rng.random() < 0.5 else 16 * int(rng.integers(1, 65))
    what = f"seed {seed}: {kv}/{qd} d={d} Hq={Hq} H={H} S={S} workers={workers} partition={part}"
    print(f"[case] {what} ctx={ctx}", flush=True)
    b = W.make_batch("random-decode", 3000 + seed, ctx, Hq, H, d, kv, qd, device=gpu,
                     pool_factor=1.3, canary=True)
    got = out_to_f64(gpu_decode(b, num_workers=workers, partition_size=part))
    e = assert_close(got, oracle_decode(b), kv, what)
    print(f"[parity] {what}: {e}", flush=True)


@pytest.mark.parametrize("seed", range(8))
def test_random_shared_prefix(gpu, seed):
    rng = np.random.default_rng(8000 + seed)
    kv, qd = TYPES[seed % len(TYPES)]
    d = (64, 128)[int(rng.integers(0, 2))]
    Hq, H = _heads(rng, d)
    S = int(rng.integers(4, 61))
    # contiguous groups with gaps of ungrouped sequences between them
    groups, s = [], int(rng.integers(0, 3))
    while s < S - 1:
        size = int(rng.integers(1, min(16, S - s) + 1))
        groups.append((s, s + size, int(rng.integers(0, 21))))
        s += size + int(rng.integers(0, 3))
    member = {i: p for a, e, p in groups for i in range(a, e)}
    ctx = [member[i] * BLOCK + int(rng.integers(0, 101)) if i in member else _length(rng)
           for i in range(S)]
    ctx = [max(c, 1) for c in ctx]
    workers = 0 if rng.random() < 0.5 else int(rng.integers(1, 301))
    what = f"seed {seed}: {kv}/{qd} d={d} Hq={Hq} H={H} S={S} groups={groups} workers={workers}"
    print(f"[case] {what}", flush=True)
    b = W.make_batch("random-shared", 4000 + seed, ctx, Hq, H, d, kv, qd, device=gpu,
                     pool_factor=1.3, prefix_groups=groups, canary=True)
    got = out_to_f64(gpu_shared_decode(b, num_workers=workers))
    e = assert_close(got, oracle_decode(b), kv, what)
    print(f"[parity] {what}: {e}", flush=True)
