"""Pins of the oracle's paged chunked-prefill attention (oracle_paged_prefill).

  * brute force: causal attention in numpy over each sequence's logical token
    list, built before the rows are scattered into a shuffled pool, for chunks
    of every kind (none, one token, part of the context, all of it);
  * closed forms: position 0 sees only itself (out = V_0); with equal K rows
    the weights are uniform over [0, p] (out = mean of V_0..V_p);
  * one query token per sequence is decode (oracle_paged_decode);
  * chunking: a prompt fed as one chunk or as several chunks (each with the
    context that precedes it) gives the same rows;
  * invalid chunk descriptions are rejected.
A planted off-by-one in the causal limit, a position counted from the chunk
start instead of the context, or a wrong query row fails the brute force.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_decode import _as_f64, scattered_case

BLOCK = 16


def brute_prefill(q, k_log, v_log, ctx, q_lens, G, scale):
    """Causal attention over the logical lists: row i of sequence s is at
    position ctx[s] - q_len + i and sees positions 0..that one."""
    T, Hq, d = q.shape
    out = np.zeros((T, Hq, d))
    qf = _as_f64(q)
    row = 0
    for s, ql in enumerate(q_lens):
        K, V = _as_f64(k_log[s]), _as_f64(v_log[s])
        for i in range(ql):
            p = ctx[s] - ql + i
            for h in range(Hq):
                x = scale * (K[: p + 1, h // G, :] @ qf[row, h])
                w = np.exp(x - x.max())
                out[row, h] = (w @ V[: p + 1, h // G, :]) / w.sum()
            row += 1
    return out


def _queries(rng, q_lens, Hq, d, like):
    from tests.test_oracle_decode import _storage
    return _storage(rng.standard_normal((int(sum(q_lens)), Hq, d)), like)


@pytest.mark.parametrize("dtype,Hq,H,d", [("f32", 4, 1, 16), ("f16", 6, 2, 32), ("bf16", 8, 8, 8)])
def test_brute_force(dtype, Hq, H, d):
    ctx = [1, 17, 40, 33, 64, 5]
    q_lens = [1, 17, 9, 0, 16, 5]   # one token, whole, part, none, a block, whole
    c = scattered_case(31, ctx, Hq, H, d, dtype)
    rng = np.random.default_rng(32)
    q = _queries(rng, q_lens, Hq, d, dtype)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    scale = 1 / np.sqrt(d)
    got = oracle.paged_prefill(q, c["k_cache"], c["v_cache"], c["bt"], c["ctx"], qs, scale)
    ref = brute_prefill(q, c["k_log"], c["v_log"], ctx, q_lens, c["G"], scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_position_zero_and_equal_keys():
    ctx = [20]
    c = scattered_case(33, ctx, 2, 1, 8, "f32")
    k = c["k_cache"].copy()
    v = c["v_cache"].copy()
    rng = np.random.default_rng(34)
    q = rng.standard_normal((20, 2, 8)).astype(np.float32)
    qs = np.array([0, 20], np.int32)
    out = oracle.paged_prefill(q, k, v, c["bt"], c["ctx"], qs, 0.3)
    V = c["v_log"][0][:, 0, :].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], V[0], rtol=0, atol=1e-15)   # sees only itself
    # every K row equal: weights uniform over [0, p]
    k[~np.isnan(k)] = 0.5
    out = oracle.paged_prefill(q, k, v, c["bt"], c["ctx"], qs, 0.3)
    for p in (0, 5, 19):
        np.testing.assert_allclose(out[p, 1], V[: p + 1].mean(axis=0), rtol=0, atol=1e-12)


def test_one_token_per_sequence_is_decode():
    ctx = [3, 16, 31, 50]
    c = scattered_case(35, ctx, 8, 2, 16, "f16")
    rng = np.random.default_rng(36)
    q = _queries(rng, [1] * 4, 8, 16, "f16")
    qs = np.arange(5, dtype=np.int32)
    got = oracle.paged_prefill(q, c["k_cache"], c["v_cache"], c["bt"], c["ctx"], qs, 0.25)
    ref = oracle.paged_decode(q, c["k_cache"], c["v_cache"], c["bt"], c["ctx"], 0.25)
    np.testing.assert_array_equal(got, ref)


def test_chunking_gives_the_same_rows():
    n = 70
    c = scattered_case(37, [n], 4, 2, 16, "bf16")
    rng = np.random.default_rng(38)
    q = _queries(rng, [n], 4, 16, "bf16")
    whole = oracle.paged_prefill(q, c["k_cache"], c["v_cache"], c["bt"], c["ctx"],
                                 np.array([0, n], np.int32), 0.2)
    rows = []
    for a, b in ((0, 23), (23, 48), (48, 70)):   # chunk [a, b) with context b
        rows.append(oracle.paged_prefill(np.ascontiguousarray(q[a:b]), c["k_cache"],
                                         c["v_cache"], c["bt"], np.array([b], np.int32),
                                         np.array([0, b - a], np.int32), 0.2))
    np.testing.assert_array_equal(np.concatenate(rows), whole)


def test_invalid_chunks_rejected():
    c = scattered_case(39, [10], 2, 1, 8, "f32")
    q = np.zeros((11, 2, 8), np.float32)
    with pytest.raises(ValueError):   # more query tokens than context
        oracle.paged_prefill(q, c["k_cache"], c["v_cache"], c["bt"], c["ctx"],
                             np.array([0, 11], np.int32), 1.0)
    with pytest.raises(ValueError):   # decreasing starts
        oracle.paged_prefill(q[:0], c["k_cache"], c["v_cache"], c["bt"], c["ctx"],
                             np.array([1, 0], np.int32), 1.0)
