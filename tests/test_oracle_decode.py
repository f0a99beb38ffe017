"""Pins of the oracle's append, gather and paged decode.

What pins what:
  * the pages' worked block-table examples (tests/golden/block_table_example.json)
    pin the slot / block reading;
  * brute force: contiguous attention in numpy over each sequence's logical
    token list, built BEFORE the rows are scattered into the pool;
  * closed forms: one token, q = 0, equal V rows, equal K rows, two tokens
    (a logistic weight), a one-hot limit, per-KV-head constant V (group map);
  * invariants: physical block permutation, shared vs copied prefix, batch
    order, split-KV vs unsplit, fp8 scale linearity;
  * NaN canaries in every row no sequence owns.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_101_amd import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "block_table_example.json")))
BLOCK = 16


# ---- helpers ---------------------------------------------------------------

def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return W.to_numpy(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    raise ValueError(dtype)


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bf16 bits
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def scattered_case(seed, ctx, Hq, H, d, dtype="f32", pool=None, shared_prefix_blocks=0,
                   max_blocks=None):
    """Logical per-sequence K/V lists, then the same rows appended into a
    shuffled pool through the oracle's append (NaN in every other row)."""
    rng = np.random.default_rng(seed)
    bps = [(max(n, 0) + BLOCK - 1) // BLOCK for n in ctx]
    need = shared_prefix_blocks + sum(max(0, b - shared_prefix_blocks) for b in bps)
    nb = pool if pool is not None else need + 3
    bt = W.assign_blocks(bps, nb, rng, shared_prefix_blocks, max_blocks)
    q = _storage(rng.standard_normal((len(ctx), Hq, d)), dtype)
    k_log, v_log = [], []
    shared_k = _storage(rng.standard_normal((shared_prefix_blocks * BLOCK, H, d)), dtype)
    shared_v = _storage(rng.standard_normal((shared_prefix_blocks * BLOCK, H, d)), dtype)
    proto = _storage(np.full((1,), np.nan), dtype)
    k_cache = np.empty((nb, H, BLOCK, d), dtype=proto.dtype)
    k_cache[...] = proto[0]
    v_cache = k_cache.copy()
    for s, n in enumerate(ctx):
        kk = _storage(rng.standard_normal((max(n, 0), H, d)), dtype)
        vv = _storage(rng.standard_normal((max(n, 0), H, d)), dtype)
        m = min(max(n, 0), shared_prefix_blocks * BLOCK)
        kk[:m] = shared_k[:m]
        vv[:m] = shared_v[:m]
        k_log.append(kk)
        v_log.append(vv)
        if n > 0:
            slots = W.slots_for_positions(bt, [s] * n, np.arange(n))
            oracle.kv_append(kk, vv, slots, k_cache, v_cache)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, bt=bt, ctx=np.array(ctx, np.int32),
                k_log=k_log, v_log=v_log, G=Hq // H)


def brute_force(q, k_log, v_log, ctx, G, scale):
    """Contiguous attention over the logical token lists, numpy float64."""
    S, Hq, d = q.shape
    out = np.zeros((S, Hq, d))
    qf = _as_f64(q)
    for s in range(S):
        if ctx[s] <= 0:
            continue
        K = _as_f64(k_log[s])  # [n][H][d]
        V = _as_f64(v_log[s])
        for h in range(Hq):
            x = scale * (K[:, h // G, :] @ qf[s, h])
            w = np.exp(x - x.max())
            out[s, h] = (w @ V[:, h // G, :]) / w.sum()
    return out


# ---- block table / append / gather -----------------------------------------

def test_worked_example_slots():
    ex = GOLD["ttlab_figure"]
    bt = np.zeros((2, 3), dtype=np.int32)
    bt[0] = ex["request_a"]["block_table"]
    bt[1, 0] = ex["request_b"]["block_table_first"]
    for pos, slot in ex["position_to_slot_a"].items():
        assert W.slots_for_positions(bt, [0], [int(pos)])[0] == slot
    for pos, slot in ex["position_to_slot_b"].items():
        assert W.slots_for_positions(bt, [1], [int(pos)])[0] == slot
    n = ex["request_a"]["tokens"]
    assert -(-n // BLOCK) == len(ex["request_a"]["block_table"])
    assert n - BLOCK * (len(ex["request_a"]["block_table"]) - 1) == ex["last_block"]["filled"]
    for r in GOLD["tarun_example"]["requests"]:
        assert -(-r["tokens"] // BLOCK) == r["blocks"]


def test_worked_example_append_fills_only_owned_rows():
    ex = GOLD["ttlab_figure"]
    n, d, H = ex["request_a"]["tokens"], 8, 1
    bt = np.array([ex["request_a"]["block_table"]], dtype=np.int32)
    k = np.arange(n * H * d, dtype=np.float32).reshape(n, H, d) + 1
    k_cache = np.full((8, H, BLOCK, d), np.nan, dtype=np.float32)
    v_cache = k_cache.copy()
    oracle.kv_append(k, -k, W.slots_for_positions(bt, [0] * n, np.arange(n)), k_cache, v_cache)
    filled = ~np.isnan(k_cache[:, 0, :, 0])
    assert filled[7].all() and filled[1].all()
    assert filled[3, :6].all() and not filled[3, 6:].any()  # physical 3 holds 6 of 16
    assert filled.sum() == n
    assert k_cache[3, 0, 5, 0] == k[37, 0, 0] and (v_cache[3, 0, 5] == -k[37, 0]).all()
    assert k_cache[7, 0, 0, 0] == k[0, 0, 0] and k_cache[1, 0, 15, 0] == k[31, 0, 0]


def test_append_negative_slot_skipped_and_out_of_range_rejected():
    k = np.ones((3, 2, 4), dtype=np.float16)
    kc = np.zeros((2, 2, BLOCK, 4), dtype=np.float16)
    vc = kc.copy()
    oracle.kv_append(k, k, np.array([-1, 5, -7]), kc, vc)
    assert kc.sum() == 8 and (kc[0, :, 5] == 1).all()
    with pytest.raises(ValueError):
        oracle.kv_append(k, k, np.array([32, 0, 1]), kc, vc)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_gather_roundtrip(dtype):
    c = scattered_case(7, [1, 15, 16, 33, 47, 0], 4, 2, 32, dtype)
    max_ctx = 48
    ko, vo = oracle.gather(c["k_cache"], c["v_cache"], c["bt"], c["ctx"], max_ctx, fill=0xAB)
    for s, n in enumerate(c["ctx"]):
        assert ko[s, :, :n].tobytes() == np.ascontiguousarray(c["k_log"][s].transpose(1, 0, 2)).tobytes()
        assert vo[s, :, :n].tobytes() == np.ascontiguousarray(c["v_log"][s].transpose(1, 0, 2)).tobytes()
        assert (ko[s, :, n:].view(np.uint8) == 0xAB).all()


# ---- decode: brute force ---------------------------------------------------

CASES = [
    ([1, 15, 16, 33], 4, 1, 64, "f32"),          # the tiny workload's shape (MQA)
    ([5, 100, 17, 64, 1], 12, 2, 128, "bf16"),   # G = 6
    ([40, 3, 129], 8, 8, 32, "f16"),             # MHA
    ([77, 31], 6, 3, 16, "f32"),                 # G = 2, odd head count
]


@pytest.mark.parametrize("ctx,Hq,H,d,dtype", CASES)
def test_decode_matches_bruteforce(ctx, Hq, H, d, dtype):
    c = scattered_case(11, ctx, Hq, H, d, dtype)
    scale = 1 / math.sqrt(d)
    got = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], scale)
    ref = brute_force(c["q"], c["k_log"], c["v_log"], c["ctx"], c["G"], scale)
    assert np.isfinite(got).all()  # NaN in every unowned row never leaks
    assert np.abs(got - ref).max() <= 1e-12


def test_tiny_workload_bruteforce_and_canaries():
    b = W.tiny(canary=True)
    kc, vc = W.to_numpy(b.k_cache), W.to_numpy(b.v_cache)
    bt, ctx = b.block_tables.numpy(), b.context_lens.numpy()
    got = oracle.paged_decode(W.to_numpy(b.q), kc, vc, bt, ctx, b.scale)
    assert np.isfinite(got).all()
    ko, vo = oracle.gather(kc, vc, bt, ctx, int(ctx.max()))
    k_log = [ko[s, :, :n].transpose(1, 0, 2) for s, n in enumerate(ctx)]
    v_log = [vo[s, :, :n].transpose(1, 0, 2) for s, n in enumerate(ctx)]
    ref = brute_force(W.to_numpy(b.q), k_log, v_log, ctx, b.group, b.scale)
    assert np.abs(got - ref).max() <= 1e-12
    assert bt.shape == (4, 3) and b.num_blocks == 16


# ---- decode: closed forms --------------------------------------------------

def _single_seq(K, V, q, scale, H=1):
    """One sequence, rows in logical order, one block per 16 positions."""
    n, d = K.shape[0], K.shape[-1]
    nb = -(-n // BLOCK) + 1
    kc = np.full((nb, H, BLOCK, d), np.nan)
    vc = kc.copy()
    kc = kc.astype(np.float32)
    vc = vc.astype(np.float32)
    bt = np.arange(1, nb, dtype=np.int32)[None, ::-1].copy()  # reversed physical order
    for t in range(n):
        kc[bt[0, t // BLOCK], :, t % BLOCK] = K[t]
        vc[bt[0, t // BLOCK], :, t % BLOCK] = V[t]
    return oracle.paged_decode(q[None].astype(np.float32), kc, vc, bt,
                               np.array([n], np.int32), scale)[0]


def test_one_token_returns_its_value():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((1, 1, 16)).astype(np.float32)
    V = rng.standard_normal((1, 1, 16)).astype(np.float32)
    q = rng.standard_normal((3, 16)).astype(np.float32) * 100
    out = _single_seq(K, V, q, 5.0)
    assert (out == V[0, 0].astype(np.float64)).all()


def test_zero_query_averages_values():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((37, 1, 8)).astype(np.float32)
    V = rng.standard_normal((37, 1, 8)).astype(np.float32)
    out = _single_seq(K, V, np.zeros((2, 8), np.float32), 1.0)
    assert np.abs(out - V[:, 0].astype(np.float64).mean(0)).max() <= 1e-14


def test_equal_values_and_equal_keys():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((20, 1, 8)).astype(np.float32)
    c = rng.standard_normal(8).astype(np.float32)
    V = np.broadcast_to(c, (20, 1, 8)).copy()
    q = rng.standard_normal((1, 8)).astype(np.float32)
    assert np.abs(_single_seq(K, V, q, 0.7) - c).max() <= 1e-14
    Keq = np.broadcast_to(K[0], (20, 1, 8)).copy()
    V2 = rng.standard_normal((20, 1, 8)).astype(np.float32)
    assert np.abs(_single_seq(Keq, V2, q, 0.7) - V2[:, 0].astype(np.float64).mean(0)).max() <= 1e-14


def test_two_tokens_logistic_weight():
    # softmax over two scores is the logistic function of their difference:
    # out = sigma(x0 - x1) v0 + (1 - sigma(x0 - x1)) v1 with x = scale * q.k
    K = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    V = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    q = np.array([[2.0, -1.0]], np.float32)
    scale = 0.5
    a = 1.0 / (1.0 + math.exp(-scale * (2.0 - (-1.0))))
    out = _single_seq(K, V, q, scale)
    assert abs(out[0, 0] - a) <= 1e-15 and abs(out[0, 1] - (1 - a)) <= 1e-15


def test_one_hot_limit_without_overflow():
    # a huge score gap: weights are exactly 0 / 1 and nothing overflows
    rng = np.random.default_rng(4)
    K = rng.standard_normal((50, 1, 16)).astype(np.float32)
    V = rng.standard_normal((50, 1, 16)).astype(np.float32)
    q = (K[23, 0] * 1.0).reshape(1, 16)
    K[23, 0] *= 3.0  # make token 23 the unique maximiser of q . k
    out = _single_seq(K, V, q, 1e4)
    assert np.isfinite(out).all()
    assert (out[0] == V[23, 0].astype(np.float64)).all()


def test_empty_and_negative_lengths_give_zero_rows():
    c = scattered_case(5, [0, 9, -3], 2, 1, 8, "f32")
    got = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.3)
    assert (got[0] == 0).all() and (got[2] == 0).all() and np.isfinite(got[1]).all()


def test_group_map_is_contiguous():
    # V constant per KV head g: query head h must return the constant of h // G
    H, G, d, n = 3, 4, 8, 21
    rng = np.random.default_rng(6)
    K = rng.standard_normal((n, H, d)).astype(np.float32)
    consts = np.arange(1, H + 1, dtype=np.float32)
    V = np.broadcast_to(consts[None, :, None], (n, H, d)).copy()
    q = rng.standard_normal((H * G, d)).astype(np.float32)
    out = _single_seq(K, V, q, 0.5, H=H)
    for h in range(H * G):
        assert np.abs(out[h] - consts[h // G]).max() <= 1e-14


def test_gqa_equals_mha_with_repeated_heads():
    c = scattered_case(8, [33, 70], 8, 2, 16, "f32")
    G = 4
    gqa = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.25)
    kc = np.repeat(c["k_cache"], G, axis=1)
    vc = np.repeat(c["v_cache"], G, axis=1)
    mha = oracle.paged_decode(c["q"], kc, vc, c["bt"], c["ctx"], 0.25)
    assert (gqa == mha).all()


# ---- decode: invariants ----------------------------------------------------

def test_physical_block_permutation_changes_nothing():
    c = scattered_case(9, [50, 16, 81], 4, 2, 16, "bf16")
    base = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.2)
    nb = c["k_cache"].shape[0]
    perm = np.random.default_rng(10).permutation(nb)  # new id of old block i is perm[i]
    kc = np.empty_like(c["k_cache"])
    vc = np.empty_like(c["v_cache"])
    kc[perm] = c["k_cache"]
    vc[perm] = c["v_cache"]
    moved = oracle.paged_decode(c["q"], kc, vc, perm[c["bt"]].astype(np.int32), c["ctx"], 0.2)
    assert (base == moved).all()


def test_shared_prefix_equals_private_copies():
    ctx = [40, 37, 64]
    c = scattered_case(12, ctx, 4, 2, 16, "f16", shared_prefix_blocks=2)
    assert (c["bt"][:, :2] == c["bt"][0, :2]).all()  # one physical copy of the prefix
    shared = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.3)
    # same logical lists, every sequence with its own blocks
    rng = np.random.default_rng(13)
    bps = [-(-n // BLOCK) for n in ctx]
    nb = sum(bps) + 1
    bt = W.assign_blocks(bps, nb, rng)
    kc = np.full((nb, 2, BLOCK, 16), np.nan, np.float16)
    vc = kc.copy()
    for s, n in enumerate(ctx):
        oracle.kv_append(c["k_log"][s], c["v_log"][s],
                         W.slots_for_positions(bt, [s] * n, np.arange(n)), kc, vc)
    private = oracle.paged_decode(c["q"], kc, vc, bt, c["ctx"], 0.3)
    assert (shared == private).all()


def test_batch_order_permutes_outputs():
    c = scattered_case(14, [20, 5, 60, 33], 2, 1, 8, "f32")
    base = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.4)
    p = np.array([2, 0, 3, 1])
    got = oracle.paged_decode(np.ascontiguousarray(c["q"][p]), c["k_cache"], c["v_cache"],
                              np.ascontiguousarray(c["bt"][p]), c["ctx"][p], 0.4)
    assert (got == base[p]).all()


@pytest.mark.parametrize("P", [16, 48, 64, 512])
def test_split_matches_unsplit(P):
    c = scattered_case(15, [1, 15, 16, 33, 100, 250], 6, 3, 16, "f32", max_blocks=20)
    ref = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.35)
    out, pm, pl, po = oracle.paged_decode_split(c["q"], c["k_cache"], c["v_cache"], c["bt"],
                                                c["ctx"], 0.35, P)
    assert np.abs(out - ref).max() <= 1e-12
    # each partition's (o_j, m_j, l_j) is the attention over its own token range
    for s, n in enumerate(c["ctx"]):
        for j in range(pm.shape[2]):
            t0 = j * P
            if t0 >= n:
                assert pl[s, :, j].max() == 0.0 and np.isneginf(pm[s, :, j]).all()
                continue
            sub_bt = np.zeros((1, c["bt"].shape[1]), np.int32)
            sub_bt[0, : c["bt"].shape[1] - t0 // BLOCK] = c["bt"][s, t0 // BLOCK:]
            sub = oracle.paged_decode(c["q"][s:s + 1], c["k_cache"], c["v_cache"], sub_bt,
                                      np.array([min(P, n - t0)], np.int32), 0.35)
            assert np.abs(po[s, :, j] - sub[0]).max() <= 1e-12
            assert (pl[s, :, j] >= 1.0).all()  # the max term contributes exp(0) = 1


def test_split_single_partition_is_identity():
    c = scattered_case(16, [30, 64], 4, 2, 8, "f16", max_blocks=4)
    ref = oracle.paged_decode(c["q"], c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.5)
    out, pm, pl, po = oracle.paged_decode_split(c["q"], c["k_cache"], c["v_cache"], c["bt"],
                                                c["ctx"], 0.5, 64)
    assert pm.shape[2] == 1
    assert np.abs(po[:, :, 0] - ref).max() <= 1e-15 and np.abs(out - ref).max() <= 1e-15


# ---- fp8 -------------------------------------------------------------------

def test_fp8_cache_equals_dequantised_float_cache():
    b = W.make_batch("t", 99, [17, 40, 1], 8, 2, 64, "fp8", "bf16", num_blocks=12)
    kc8, vc8 = W.to_numpy(b.k_cache), W.to_numpy(b.v_cache)
    bt, ctx, q = b.block_tables.numpy(), b.context_lens.numpy(), W.to_numpy(b.q)
    got = oracle.paged_decode(q, kc8, vc8, bt, ctx, b.scale, b.k_scale, b.v_scale)
    kf = (b.k_cache.view(torch.float8_e4m3fn).to(torch.float64) * b.k_scale).numpy()
    vf = (b.v_cache.view(torch.float8_e4m3fn).to(torch.float64) * b.v_scale).numpy()
    # float64 copies of code * scale are exact, so a float64 attention over
    # them (the brute force) must agree to rounding
    ko = [kf[bt[s, np.arange(n) // 16], :, np.arange(n) % 16] for s, n in enumerate(ctx)]
    vo = [vf[bt[s, np.arange(n) // 16], :, np.arange(n) % 16] for s, n in enumerate(ctx)]
    ref = brute_force(q, ko, vo, ctx, b.group, b.scale)
    assert np.abs(got - ref).max() <= 1e-12
    # scale linearity: doubling k_scale is doubling the softmax scale,
    # doubling v_scale doubles the output
    a = oracle.paged_decode(q, kc8, vc8, bt, ctx, b.scale, 2 * b.k_scale, b.v_scale)
    bb = oracle.paged_decode(q, kc8, vc8, bt, ctx, 2 * b.scale, b.k_scale, b.v_scale)
    assert np.abs(a - bb).max() <= 1e-12
    c2 = oracle.paged_decode(q, kc8, vc8, bt, ctx, b.scale, b.k_scale, 2 * b.v_scale)
    assert np.abs(c2 - 2 * got).max() <= 1e-12
