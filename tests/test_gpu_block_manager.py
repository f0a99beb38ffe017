"""GPU: the host block manager driving the device path end to end.

Requests with a common system prompt (prefix-cache hits), a unique one, and a
forked request whose children write into a shared partial block
(copy-on-write) go through the manager; its slot mappings feed pkv_kv_append,
its copies pkv_copy_blocks, its block tables and prefix groups plain and
shared-prefix decode. The expected side is built on the host alone: every
token's K/V rows are a function of the token sequence up to it (so requests
that share a prefix share its rows, as a model would give them), placed by
the manager's final block tables into row-order caches for the oracle.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_101_amd import binding as B
from paged_kv_cache_101_amd import workloads as W
from paged_kv_cache_101_amd.blocks import BlockManager
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
BS = 16
H, HQ, D = 8, 32, 128


def rows_for(history):
    """K and V rows [2][H][D] (bf16 as float32 values) of the last token of a
    token history: seeded by the whole history."""
    seed = int.from_bytes(hashlib.blake2b(np.asarray(history, dtype=np.int64).tobytes(),
                                          digest_size=8).digest(), "little")
    x = np.random.default_rng(seed).standard_normal((2, H, D)).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_manager_append_copy_decode(gpu):
    nb = 160
    bm = BlockManager(nb)
    kc = torch.zeros((nb, H, BS, D), dtype=torch.bfloat16, device=gpu)
    vc = torch.zeros_like(kc)
    desc = B.desc_for(kc, "bf16")
    hist = {}

    def push(rid, n, new=None):
        """Slots for n tokens of rid, copy-on-write first, then the append."""
        slots, copies = bm.append(rid, n, new)
        if copies.size:
            B.pkv_copy_blocks(kc, vc, desc, torch.from_numpy(copies).to(gpu))
        toks = hist[rid]
        start = len(toks) - n
        kv = np.stack([rows_for(toks[: start + i + 1]) for i in range(n)])  # [n][2][H][D]
        kv = torch.from_numpy(kv).to(torch.bfloat16).to(gpu)
        B.pkv_kv_append(kv[:, 0].contiguous(), kv[:, 1].contiguous(),
                        torch.from_numpy(slots).to(gpu), kc, vc, desc)

    rng = np.random.default_rng(5)
    system = list(rng.integers(0, 30000, 100))
    prompts = {r: system + list(rng.integers(0, 30000, int(rng.integers(20, 61))))
               for r in range(6)}
    prompts[6] = list(rng.integers(0, 30000, 77))
    hits = {}
    for r, p in prompts.items():
        hits[r] = bm.add_request(r, p)
        hist[r] = list(p)
        push(r, len(p) - hits[r])
    assert hits[0] == 0 and all(hits[r] == 96 for r in range(1, 6)) and hits[6] == 0
    # parallel sampling: request 6 forks twice; the children write into the
    # shared partial block (77 tokens: 13 of 16 in the last block)
    for child in (7, 8):
        bm.fork(6, child)
        hist[child] = list(hist[6])
    for step in range(3):
        for r in range(9):
            t = int(rng.integers(0, 30000))
            hist[r].append(t)
            push(r, 1, [t])
    torch.cuda.synchronize()

    # order the batch so that sharers are adjacent: 0-5, then 6-8
    ids = list(range(9))
    mb = 16
    bt, cl = bm.block_tables(ids, mb)
    assert (cl == np.array([len(hist[r]) for r in ids])).all()
    assert len({int(bt[r, 4]) for r in (6, 7, 8)}) == 3      # copy-on-write gave each its own
    starts, pre = bm.prefix_groups(ids)
    assert starts.tolist() == [0, 6, 9] and pre.tolist() == [6, 4]

    # the expected row-order caches, from the host alone
    ek = np.full((nb, H, BS, D), np.nan, dtype=np.float32)
    ev = ek.copy()
    for i, r in enumerate(ids):
        for p in range(len(hist[r])):
            kv = rows_for(hist[r][: p + 1])
            ek[bt[i, p // BS], :, p % BS] = kv[0]
            ev[bt[i, p // BS], :, p % BS] = kv[1]
    ek16 = torch.from_numpy(ek).to(torch.bfloat16)
    ev16 = torch.from_numpy(ev).to(torch.bfloat16)
    # the device caches hold exactly those rows (unused rows aside)
    gk, gv = B.read_cache(kc, vc, desc)
    used = ~torch.isnan(ek16[:, 0, :, 0])  # [block][row]
    rows = lambda t: t.permute(0, 2, 1, 3)[used]  # noqa: E731  (used rows, every head)
    assert torch.equal(rows(gk.cpu()), rows(ek16)) and torch.equal(rows(gv.cpu()), rows(ev16))

    q = torch.randn((len(ids), HQ, D), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    ref = oracle.paged_decode(W.to_numpy(q), W.to_numpy(ek16), W.to_numpy(ev16), bt, cl, scale)
    qd = q.to(gpu)
    btd = torch.from_numpy(bt).to(gpu)
    cld = torch.from_numpy(cl).to(gpu)
    out = torch.empty_like(qd)
    B.pkv_paged_attention_decode(qd, kc, vc, desc, btd, cld, scale, out)
    assert_close(out.double().cpu().numpy(), ref, "bf16", "plain decode")
    out2 = torch.empty_like(qd)
    B.pkv_paged_attention_decode_shared_prefix(qd, kc, vc, desc, btd, cld,
                                               torch.from_numpy(starts).to(gpu),
                                               torch.from_numpy(pre).to(gpu), scale, out2)
    assert_close(out2.double().cpu().numpy(), ref, "bf16", "shared-prefix decode")


def test_copy_blocks_bytes(gpu):
    nb, Hh, d = 12, 4, 64
    kc = torch.randn((nb, Hh, BS, d), device=gpu).to(torch.float16)
    vc = torch.randn((nb, Hh, BS, d), device=gpu).to(torch.float16)
    desc = B.desc_for(kc, "f16")
    before_k, before_v = kc.clone(), vc.clone()
    pairs = torch.tensor([[3, 7], [5, 1], [0, 11], [4, 12], [-1, 2]], dtype=torch.int32,
                         device=gpu)  # the last two are outside the pool: skipped
    B.pkv_copy_blocks(kc, vc, desc, pairs)
    torch.cuda.synchronize()
    ek, ev = before_k.clone(), before_v.clone()
    for s, d_ in ((3, 7), (5, 1), (0, 11)):
        ek[d_], ev[d_] = before_k[s], before_v[s]
    assert torch.equal(kc, ek) and torch.equal(vc, ev)
