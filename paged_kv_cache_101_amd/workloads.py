"""Seeded synthetic inputs for paged decode attention.

This module only builds inputs: sequence lengths, a physical block pool with
its block tables, slot mappings for new tokens, and N(0,1) values cast to the
storage dtype. It holds none of the attention arithmetic, so both the GPU
tests and the CPU oracle can be fed from it.

Recipe
  * Structure (lengths, the permutation of physical blocks) comes from
    ``numpy.random.default_rng([case_id, stream, layer])`` with stream 0 for
    lengths and stream 1 for the block permutation.
  * Values come from a ``torch.Generator`` on the target device, seeded from
    (case_id, stream, layer) with stream 2 = q, 3 = K, 4 = V, 5 = new K/V rows.
    They are N(0,1) float32 rounded to nearest-even into the storage dtype.
  * Physical block 0 is the reserved null block (the ttlab page, section 4,
    keeps block 0 out of the free queue). Block-table entries past a
    sequence's last block point at it. The remaining ids are a random
    permutation handed out in logical order (seq 0 block 0, seq 0 block 1, ...).
  * A slot is phys * 16 + position % 16 (row position % 16 of the block that
    holds the position).
  * ``canary=True`` fills every cache row no sequence uses (the tail of a
    partly filled block, free pool blocks, the null block) with NaN, and the
    row a pending append will write, so that reading any of them shows up.
  * fp8 (OCP E4M3FN) caches use one scale per tensor, max|x| / 448 over the
    rows in use, and store round-to-nearest-even(clamp(x / scale, +-448)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 16
FP8_MAX = 448.0
FP8_NAN = 0x7F

# storage dtype name -> (torch dtype used to hold it, bytes per element)
STORAGE = {
    "f32": (torch.float32, 4),
    "f16": (torch.float16, 2),
    "bf16": (torch.bfloat16, 2),
    "fp8": (torch.uint8, 1),
}


def _seed(case_id: int, stream: int, layer: int) -> int:
    return (case_id * 1_000_003 + stream * 10_007 + layer * 101 + 12345) % (2**63 - 1)


def _gen(device, case_id, stream, layer):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(case_id, stream, layer))
    return g


def _randn(shape, device, case_id, stream, layer):
    return torch.randn(shape, generator=_gen(device, case_id, stream, layer), device=device,
                       dtype=torch.float32)


def to_storage(x: torch.Tensor, dtype: str, scale: float = 1.0) -> torch.Tensor:
    """Round float32 values into a storage dtype (fp8: codes of x / scale)."""
    if dtype == "fp8":
        y = torch.clamp(x / scale, -FP8_MAX, FP8_MAX)
        return y.to(torch.float8_e4m3fn).view(torch.uint8)
    return x.to(STORAGE[dtype][0])


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a storage tensor in the layout the oracle reads (bf16 as
    raw uint16 bits, fp8 as raw uint8 codes)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class DecodeBatch:
    """One paged decode call's inputs (and optional pending appends)."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    q_dtype: str
    num_blocks: int
    context_lens: torch.Tensor          # int32 [S]
    block_tables: torch.Tensor          # int32 [S][max_blocks]
    q: torch.Tensor                     # [S][H_q][d]
    k_cache: torch.Tensor               # [num_blocks][H_kv][16][d]
    v_cache: torch.Tensor
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    new_k: Optional[torch.Tensor] = None   # [T][H_kv][d]
    new_v: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None  # int64 [T]
    # fp8 caches only: the new rows before quantisation, in the query's
    # 16-bit type, for a quantising append (new_k / new_v hold their codes)
    new_k_rows: Optional[torch.Tensor] = None
    new_v_rows: Optional[torch.Tensor] = None
    # prefix groups: sequences [starts[j], starts[j+1]) share their first
    # prefix[j] blocks (None: no description)
    group_starts: Optional[torch.Tensor] = None  # int32 [G + 1]
    group_prefix: Optional[torch.Tensor] = None  # int32 [G]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes(self) -> int:
        """Bytes of K and V the batch attends over (every sequence counted)."""
        b = STORAGE[self.kv_dtype][1]
        n = int(self.context_lens.clamp(min=0).sum())
        return n * 2 * self.num_kv_heads * self.head_dim * b


def group_prefix_of(num_seqs: int, groups) -> np.ndarray:
    """Shared blocks of each sequence under a list of (start, end, blocks)."""
    pre = np.zeros(num_seqs, dtype=np.int64)
    for a, b, p in groups:
        pre[a:b] = p
    return pre


def group_arrays(groups):
    """The library's description of (start, end, blocks) groups: group j is
    sequences [starts[j], starts[j + 1]), so groups are adjacent runs; a gap
    between two groups becomes a group with no shared blocks."""
    starts, prefix, end = [], [], None
    for a, b, p in sorted(groups):
        if end is not None and a > end:
            starts.append(end)
            prefix.append(0)
        starts.append(a)
        prefix.append(p)
        end = b
    if end is not None:
        starts.append(end)
    return starts, prefix


def blocks_needed(blocks_per_seq: Sequence[int], groups) -> int:
    """Physical blocks a batch uses: each group's prefix once, plus every
    sequence's own blocks."""
    pre = group_prefix_of(len(blocks_per_seq), groups)
    return int(sum(p for _, _, p in groups) +
               sum(max(0, b - pre[s]) for s, b in enumerate(blocks_per_seq)))


def assign_blocks(blocks_per_seq: Sequence[int], num_blocks: int, rng: np.random.Generator,
                  shared_prefix_blocks: int = 0, max_blocks: Optional[int] = None,
                  groups=None):
    """Block tables from a shuffled pool; block 0 is the null block.

    ``groups`` lists (start, end, P): sequences [start, end) map their first P
    logical blocks to the same P physical blocks (one copy of a common
    prefix). ``shared_prefix_blocks`` is the one-group case over every
    sequence. Each group's blocks are handed out first, in group order."""
    S = len(blocks_per_seq)
    if groups is None:
        groups = [(0, S, shared_prefix_blocks)] if shared_prefix_blocks else []
    mb = max_blocks if max_blocks is not None else max(1, max(blocks_per_seq))
    need = blocks_needed(blocks_per_seq, groups)
    if need > num_blocks - 1:
        raise ValueError(f"pool of {num_blocks} blocks too small for {need} (+1 null)")
    ids = rng.permutation(np.arange(1, num_blocks, dtype=np.int64))
    bt = np.zeros((S, mb), dtype=np.int32)
    nxt = 0
    for a, b, p in groups:
        shared = ids[nxt:nxt + p]
        nxt += p
        for s in range(a, b):
            n = min(p, blocks_per_seq[s])
            bt[s, :n] = shared[:n]
    pre = group_prefix_of(S, groups)
    for s, nb in enumerate(blocks_per_seq):
        for i in range(int(pre[s]), nb):
            bt[s, i] = ids[nxt]
            nxt += 1
    return bt


def slots_for_positions(block_tables: np.ndarray, seq_ids, positions) -> np.ndarray:
    """Slot of (sequence, position): phys * 16 + position % 16."""
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    phys = block_tables[seq_ids, positions // BLOCK].astype(np.int64)
    return phys * BLOCK + positions % BLOCK


def used_rows_per_block(block_tables: np.ndarray, context_lens: np.ndarray, num_blocks: int):
    """Number of leading rows of each physical block that some sequence reads."""
    used = np.zeros(num_blocks, dtype=np.int64)
    for s in range(block_tables.shape[0]):
        n = int(context_lens[s])
        for i in range((max(n, 0) + BLOCK - 1) // BLOCK):
            p = int(block_tables[s, i])
            used[p] = max(used[p], min(BLOCK, n - i * BLOCK))
    return used


def make_batch(name: str, case_id: int, context_lens: Sequence[int], num_q_heads: int,
               num_kv_heads: int, head_dim: int, kv_dtype: str, q_dtype: str,
               device="cpu", layer: int = 0, num_blocks: Optional[int] = None,
               pool_factor: float = 1.0, shared_prefix_blocks: int = 0,
               prefix_groups=None,
               max_blocks: Optional[int] = None, canary: bool = False,
               append_last: bool = False,
               scale: Optional[float] = None, structure_layer: Optional[int] = None) -> DecodeBatch:
    """Build one decode batch.

    ``append_last`` holds back the K/V row at position n-1 of every sequence
    with n > 0: its slot is left as NaN (canary) or random, and the row to
    write comes back in ``new_k``/``new_v``/``slot_mapping`` for an append
    call made before decode. ``structure_layer`` (default: ``layer``) seeds the
    block permutation, so several layers can share one block table."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.shape[0]
    bps = [(max(int(n), 0) + BLOCK - 1) // BLOCK for n in ctx]
    mb = max_blocks if max_blocks is not None else max(1, max(bps) if bps else 1)
    if prefix_groups is None:
        prefix_groups = [(0, S, shared_prefix_blocks)] if shared_prefix_blocks else []
    prefix_groups = [(int(a), int(b), int(p)) for a, b, p in prefix_groups]
    need = blocks_needed(bps, prefix_groups)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need)) + 1
    rng = np.random.default_rng([case_id, 1, layer if structure_layer is None else structure_layer])
    bt = assign_blocks(bps, num_blocks, rng, max_blocks=mb, groups=prefix_groups)

    H, d = num_kv_heads, head_dim
    cache_shape = (num_blocks, H, BLOCK, d)
    kx = _randn(cache_shape, device, case_id, 3, layer)
    vx = _randn(cache_shape, device, case_id, 4, layer)
    qx = _randn((S, num_q_heads, d), device, case_id, 2, layer)

    used = used_rows_per_block(bt, ctx, num_blocks)
    row_used = torch.from_numpy(np.arange(BLOCK)[None, :] < used[:, None]).to(device)
    row_used = row_used[:, None, :, None]  # [nb][1][16][1]

    new_k = new_v = slot_mapping = None
    pending = None
    if append_last:
        seqs = [s for s in range(S) if ctx[s] > 0]
        slots = slots_for_positions(bt, seqs, [ctx[s] - 1 for s in seqs])
        pending = torch.zeros((num_blocks * BLOCK,), dtype=torch.bool)
        pending[torch.from_numpy(slots)] = True
        pending = pending.view(num_blocks, 1, BLOCK, 1).to(device)
        nk = _randn((len(seqs), H, d), device, case_id, 5, layer)
        nv = _randn((len(seqs), H, d), device, case_id, 5, layer + 7919)
        slot_mapping = torch.from_numpy(slots.astype(np.int64)).to(device)

    k_scale = v_scale = 1.0
    if kv_dtype == "fp8":
        rows = row_used if pending is None else row_used
        k_scale = float(kx.abs().masked_fill(~rows, 0).amax()) / FP8_MAX
        v_scale = float(vx.abs().masked_fill(~rows, 0).amax()) / FP8_MAX
        if append_last:
            k_scale = max(k_scale, float(nk.abs().amax()) / FP8_MAX)
            v_scale = max(v_scale, float(nv.abs().amax()) / FP8_MAX)

    k_cache = to_storage(kx, kv_dtype, k_scale)
    v_cache = to_storage(vx, kv_dtype, v_scale)
    del kx, vx
    if canary:
        poison = ~row_used
        if pending is not None:
            poison = poison | pending
        nan = FP8_NAN if kv_dtype == "fp8" else float("nan")
        k_cache.masked_fill_(poison.expand_as(k_cache), nan)
        v_cache.masked_fill_(poison.expand_as(v_cache), nan)
    new_k_rows = new_v_rows = None
    if append_last:
        new_k = to_storage(nk, kv_dtype, k_scale)
        new_v = to_storage(nv, kv_dtype, v_scale)
        if kv_dtype == "fp8":
            new_k_rows = nk.to(STORAGE[q_dtype][0])
            new_v_rows = nv.to(STORAGE[q_dtype][0])

    q = qx.to(STORAGE[q_dtype][0])
    starts, prefix = group_arrays(prefix_groups)
    return DecodeBatch(
        name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        kv_dtype=kv_dtype, q_dtype=q_dtype, num_blocks=num_blocks,
        context_lens=torch.from_numpy(ctx.astype(np.int32)).to(device),
        block_tables=torch.from_numpy(bt).to(device), q=q, k_cache=k_cache, v_cache=v_cache,
        scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
        k_scale=k_scale, v_scale=v_scale,
        new_k=new_k, new_v=new_v, slot_mapping=slot_mapping, new_k_rows=new_k_rows,
        new_v_rows=new_v_rows,
        group_starts=(torch.tensor(starts, dtype=torch.int32, device=device)
                      if prefix_groups else None),
        group_prefix=(torch.tensor(prefix, dtype=torch.int32, device=device)
                      if prefix_groups else None),
        meta={"case_id": case_id, "layer": layer, "shared_prefix_blocks": shared_prefix_blocks,
              "prefix_groups": prefix_groups})


# ---- the five workloads ----------------------------------------------------

def tiny(device="cpu", canary=False) -> DecodeBatch:
    """4 sequences of lengths {1, 15, 16, 33}; 4 query heads on 1 KV head
    (MQA), d 64, fp32, a pool of 16 blocks."""
    return make_batch("tiny", 1, [1, 15, 16, 33], 4, 1, 64, "f32", "f32", device=device,
                      num_blocks=16, canary=canary)


def qwen_layer_lengths(num_seqs=64, lo=128, hi=4096, case_id=2):
    rng = np.random.default_rng([case_id, 0, 0])
    return rng.integers(lo, hi + 1, size=num_seqs)


def qwen_layer(device="cpu", canary=False, num_seqs=64, lo=128, hi=4096) -> DecodeBatch:
    """Qwen2.5-1.5B-shaped layer: 12 query / 2 KV heads, d 128, bf16 KV,
    64 sequences with lengths uniform in [128, 4096], a pool 1.5x the blocks
    needed, and one appended token per sequence (its position is n-1)."""
    ctx = qwen_layer_lengths(num_seqs, lo, hi)
    return make_batch("qwen2.5-1.5b-layer", 2, ctx, 12, 2, 128, "bf16", "bf16", device=device,
                      pool_factor=1.5, canary=canary, append_last=True)


def gqa40_layer(device="cpu", layer=0, num_seqs=40, ctx=8192, canary=False,
                append_last=False) -> DecodeBatch:
    """One layer of the 40-layer GQA shape: 32 query / 8 KV heads, d 128,
    fp16 KV, 40 sequences of 8192 tokens, shuffled blocks. Every layer has its
    own caches and queries; all layers share one block table."""
    return make_batch("gqa40-8k", 3, [ctx] * num_seqs, 32, 8, 128, "f16", "f16", device=device,
                      layer=layer, canary=canary, append_last=append_last, structure_layer=0)


def gqa40_tp8_layer(device="cpu", layer=0, num_seqs=40, ctx=8192, canary=False,
                    append_last=False) -> DecodeBatch:
    """One GPU's share of a layer of the 40-layer GQA shape when its 8 KV heads
    are split over 8 GPUs (tensor parallel over heads): 4 query / 1 KV head,
    d 128, fp16 KV, 40 sequences of 8192 tokens; all layers share one block
    table."""
    return make_batch("gqa40-8k-tp8", 6, [ctx] * num_seqs, 4, 1, 128, "f16", "f16", device=device,
                      layer=layer, canary=canary, append_last=append_last, structure_layer=0)


def prefix_shared_lengths(num_seqs=256, prefix=2048, lo=64, hi=512, case_id=4):
    rng = np.random.default_rng([case_id, 0, 0])
    suf = rng.integers(lo, hi + 1, size=num_seqs)
    while np.any(suf % BLOCK == 0):
        redraw = suf % BLOCK == 0
        suf[redraw] = rng.integers(lo, hi + 1, size=int(redraw.sum()))
    return prefix + suf


def prefix_shared(device="cpu", canary=False, num_seqs=256, prefix=2048) -> DecodeBatch:
    """256 sequences sharing a 2048-token prefix (128 physical blocks, one copy)
    plus a private suffix of 64-512 tokens ending in a partly filled block;
    32 query / 8 KV heads, d 128, bf16."""
    ctx = prefix_shared_lengths(num_seqs, prefix)
    return make_batch("prefix-shared", 4, ctx, 32, 8, 128, "bf16", "bf16", device=device,
                      shared_prefix_blocks=prefix // BLOCK, canary=canary,
                      max_blocks=(prefix + 512 + BLOCK - 1) // BLOCK)


def fp8_long(device="cpu", canary=False, num_seqs=16, ctx=32768,
             append_last=False) -> DecodeBatch:
    """16 sequences of 32768 tokens, 64 query / 8 KV heads, d 128, fp8 E4M3FN
    KV with one scale per tensor, bf16 q/out. ``append_last`` holds back each
    sequence's last row for a quantising append of bf16 rows."""
    return make_batch("fp8-long", 5, [ctx] * num_seqs, 64, 8, 128, "fp8", "bf16", device=device,
                      canary=canary, append_last=append_last)
