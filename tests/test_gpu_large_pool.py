"""GPU: a KV pool larger than 4 GiB per cache. The blocks a batch uses sit
below, across and far past the 4 GiB mark (fp16, 8 KV heads, d 128: 32 KiB
per block and cache, so block 131072 starts at byte 2^32), so every tile's
byte offset into the pool needs more than 32 bits.

The rows are written into the pool with pkv_kv_append, then decode, chunked
prefill (with and without the split workspace) and the shared-prefix decode
read them back. The oracle reads a compact copy holding only the used blocks,
renumbered: where a block sits in the pool does not enter the computation.
Unused pool memory holds NaN, so a read from a wrong place shows."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_101_amd import binding as B
from tests.helpers import assert_close, out_to_f64

pytestmark = pytest.mark.gpu

BLOCK = 16
NUM_BLOCKS = 140_000          # 140000 * 32 KiB = 4.59e9 bytes per cache
HQ, H, D = 32, 8, 128
PLAIN_CTX = [1, 17, 300, 1000, 2049, 4096]
PREFIX_BLOCKS = 64            # the group shares the first 64 blocks of the 4096-token sequence
MEMBER_SUFFIX = [1, 15, 16, 40, 100]


@pytest.fixture(scope="module")
def pool(gpu):
    free, _ = torch.cuda.mem_get_info()
    need = 2 * NUM_BLOCKS * H * BLOCK * D * 2
    assert free > need + (2 << 30), f"needs {need / 2**30:.1f} GiB of device memory"
    rng = np.random.default_rng(71)
    # block ids: just above the null block, around the 4 GiB boundary, and at the top
    ids = np.concatenate([np.arange(1, 120), np.arange(131_000, 131_200),
                          np.arange(NUM_BLOCKS - 300, NUM_BLOCKS)])
    ids = rng.permutation(ids)
    nxt = iter(ids.tolist())

    plain_bt = [[next(nxt) for _ in range(-(-n // BLOCK))] for n in PLAIN_CTX]
    shared = plain_bt[5][:PREFIX_BLOCKS]
    member_ctx = [PREFIX_BLOCKS * BLOCK + m for m in MEMBER_SUFFIX]
    member_bt = [shared + [next(nxt) for _ in range(-(-m // BLOCK))] for m in MEMBER_SUFFIX]
    tables = plain_bt + member_bt
    ctx = PLAIN_CTX + member_ctx
    S = len(tables)
    mb = max(len(t) for t in tables)
    bt = np.zeros((S, mb), dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t

    # token rows: a plain sequence writes all its tokens, a group member only
    # its suffix (its prefix rows are the 4096-token sequence's)
    slots, owners = [], []
    for s in range(S):
        first = PREFIX_BLOCKS * BLOCK if s >= len(PLAIN_CTX) else 0
        for p in range(first, ctx[s]):
            slots.append(bt[s, p // BLOCK] * BLOCK + p % BLOCK)
            owners.append((s, p))
    T = len(slots)
    k_rows = rng.standard_normal((T, H, D)).astype(np.float16)
    v_rows = rng.standard_normal((T, H, D)).astype(np.float16)

    k_cache = torch.full((NUM_BLOCKS, H, BLOCK, D), float("nan"), dtype=torch.float16, device=gpu)
    v_cache = torch.full_like(k_cache, float("nan"))
    desc = B.desc_for(k_cache, "f16")
    B.pkv_kv_append(torch.from_numpy(k_rows).to(gpu), torch.from_numpy(v_rows).to(gpu),
                    torch.tensor(slots, dtype=torch.int64, device=gpu), k_cache, v_cache, desc)

    # the oracle's compact copy: used blocks renumbered 0..U-1
    used = np.unique(bt[bt > 0])
    local = {int(b): i for i, b in enumerate(used)}
    kh = np.zeros((len(used), H, BLOCK, D), dtype=np.float16)
    vh = np.zeros_like(kh)
    for i, slot in enumerate(slots):
        blk, row = divmod(slot, BLOCK)
        kh[local[blk], :, row, :] = k_rows[i]
        vh[local[blk], :, row, :] = v_rows[i]
    bt_local = np.zeros_like(bt)
    for s, t in enumerate(tables):
        bt_local[s, :len(t)] = [local[b] for b in t]
    torch.cuda.synchronize()
    return dict(k_cache=k_cache, v_cache=v_cache, desc=desc, bt=bt, bt_local=bt_local,
                ctx=np.array(ctx, dtype=np.int32), kh=kh, vh=vh, S=S, rng=rng)


def test_pool_spans_past_4gib(pool):
    assert pool["k_cache"].numel() * 2 > 2**32
    top = int(pool["bt"].max())
    assert top * H * BLOCK * D * 2 > 2**32  # a used tile starts past byte 2^32


def test_decode(pool, gpu):
    S = pool["S"]
    q = torch.from_numpy(pool["rng"].standard_normal((S, HQ, D)).astype(np.float16)).to(gpu)
    out = torch.empty_like(q)
    scale = D ** -0.5
    B.pkv_paged_attention_decode(q, pool["k_cache"], pool["v_cache"], pool["desc"],
                                 torch.from_numpy(pool["bt"]).to(gpu),
                                 torch.from_numpy(pool["ctx"]).to(gpu), scale, out)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(q.cpu().numpy(), pool["kh"], pool["vh"], pool["bt_local"],
                              pool["ctx"], scale)
    e = assert_close(out_to_f64(out), ref, "f16", "decode, pool past 4 GiB")
    print(f"[parity] large pool decode: {e}", flush=True)


def test_shared_prefix_decode(pool, gpu):
    S = pool["S"]
    q = torch.from_numpy(pool["rng"].standard_normal((S, HQ, D)).astype(np.float16)).to(gpu)
    out = torch.empty_like(q)
    scale = D ** -0.5
    n_plain = len(PLAIN_CTX)
    gs = torch.tensor([n_plain, S], dtype=torch.int32, device=gpu)
    gp = torch.tensor([PREFIX_BLOCKS], dtype=torch.int32, device=gpu)
    B.pkv_paged_attention_decode_shared_prefix(
        q, pool["k_cache"], pool["v_cache"], pool["desc"], torch.from_numpy(pool["bt"]).to(gpu),
        torch.from_numpy(pool["ctx"]).to(gpu), gs, gp, scale, out)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(q.cpu().numpy(), pool["kh"], pool["vh"], pool["bt_local"],
                              pool["ctx"], scale)
    e = assert_close(out_to_f64(out), ref, "f16", "shared-prefix decode, pool past 4 GiB")
    print(f"[parity] large pool shared-prefix decode: {e}", flush=True)


@pytest.mark.parametrize("split", [False, True])
def test_prefill(pool, gpu, split):
    """The last q_len tokens of each plain sequence as a chunk (a chunk over a
    long context with few rows takes the split path when a workspace is given)."""
    q_lens = [1, 17, 64, 100, 33, 200]
    n_plain = len(PLAIN_CTX)
    T = sum(q_lens)
    q = torch.from_numpy(pool["rng"].standard_normal((T, HQ, D)).astype(np.float16)).to(gpu)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out = torch.empty_like(q)
    scale = D ** -0.5
    bt = pool["bt"][:n_plain]
    ctx = pool["ctx"][:n_plain]
    ws = B.prefill_workspace(D, gpu) if split else None
    B.pkv_paged_attention_prefill(q, pool["k_cache"], pool["v_cache"], pool["desc"],
                                  torch.from_numpy(np.ascontiguousarray(bt)).to(gpu),
                                  torch.from_numpy(ctx).to(gpu), torch.from_numpy(qs).to(gpu),
                                  scale, out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.paged_prefill(q.cpu().numpy(), pool["kh"], pool["vh"],
                               pool["bt_local"][:n_plain], ctx, qs, scale)
    e = assert_close(out_to_f64(out), ref, "f16", f"prefill split={split}, pool past 4 GiB")
    print(f"[parity] large pool prefill split={split}: {e}", flush=True)
