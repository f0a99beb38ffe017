"""Pins of the oracle's quantising append into an fp8 cache.

The code of an element is that of the float32 quotient x / scale:
  * with a power-of-two scale the quotient is exact, so the float32-quotient
    encoder must equal the double-quotient encoder, itself pinned exhaustively
    against torch's cast (test_oracle_codecs.py) -- checked for every finite
    fp16 value;
  * for general scales the quotient is checked against numpy's own float32
    division, and a case where float32 and double quotients round to
    different codes shows that the float32 one decides;
  * the append places each element's code exactly where the plain byte
    append puts a row, skips negative slots and rejects slots past the pool.
"""
import numpy as np
import pytest
import torch

import oracle

BLOCK = 16


def test_encode_f32_equals_encode_for_power_of_two_scales():
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = vals[np.isfinite(vals)].astype(np.float64)
    for c in (1.0, 0.25, 4.0):
        for x in vals[::7]:
            assert oracle.fp8_e4m3_encode_f32(x, c) == oracle.fp8_e4m3_encode(x, c), (x, c)


def test_encode_f32_uses_the_float32_quotient():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * 3).astype(np.float32)
    c = rng.uniform(0.01, 1.0, 20000).astype(np.float32)
    y = x / c  # numpy float32 division (IEEE single precision)
    for xi, ci, yi in zip(x, c, y):
        assert oracle.fp8_e4m3_encode_f32(float(xi), float(ci)) == \
            oracle.fp8_e4m3_encode(float(yi), 1.0), (xi, ci)


def test_float32_and_double_quotients_can_decide_differently():
    # x / c placed on a rounding midpoint between two codes: the float32 and
    # the double quotient then fall on different sides of it for some pairs
    rng = np.random.default_rng(12)
    found = 0
    for _ in range(40000):
        c = np.float32(rng.uniform(0.003, 0.9))
        mid = 1.0625 * 2.0 ** int(rng.integers(-5, 8))  # midway between 1 and 1 + 1/8
        x = np.float32(mid * float(c))
        dbl = oracle.fp8_e4m3_encode(float(x), float(c))
        f32 = oracle.fp8_e4m3_encode(float(x / c), 1.0)
        if dbl != f32:
            assert oracle.fp8_e4m3_encode_f32(float(x), float(c)) == f32
            found += 1
    assert found > 0


def _rows(dtype, shape, rng):
    x = (rng.standard_normal(shape) * 2).astype(np.float32)
    if dtype == "f32":
        return x, x
    if dtype == "f16":
        h = x.astype(np.float16)
        return h, h.astype(np.float32)
    b = torch.from_numpy(x).to(torch.bfloat16)
    return b.view(torch.int16).numpy().view(np.uint16), b.to(torch.float32).numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_fp8_places_each_code_like_the_byte_append(dtype):
    rng = np.random.default_rng(13)
    T, H, d, nb = 9, 2, 64, 6
    k, kf = _rows(dtype, (T, H, d), rng)
    v, vf = _rows(dtype, (T, H, d), rng)
    slots = rng.permutation(nb * BLOCK)[:T].astype(np.int64)
    slots[3] = -1
    ks, vs = 0.0375, 0.71
    kc = np.full((nb, H, BLOCK, d), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    oracle.kv_append_fp8(k, v, slots, kc, vc, ks, vs)
    # the expected codes, element by element, placed by the plain byte append
    kcode = np.array([oracle.fp8_e4m3_encode(float(t), 1.0) for t in (kf / np.float32(ks)).ravel()],
                     dtype=np.uint8).reshape(T, H, d)
    vcode = np.array([oracle.fp8_e4m3_encode(float(t), 1.0) for t in (vf / np.float32(vs)).ravel()],
                     dtype=np.uint8).reshape(T, H, d)
    ke = np.full_like(kc, 0x7F)
    ve = ke.copy()
    oracle.kv_append(kcode, vcode, slots, ke, ve)
    assert kc.tobytes() == ke.tobytes() and vc.tobytes() == ve.tobytes()
    assert (kc == 0x7F).sum() >= (nb * BLOCK - (T - 1)) * H * d  # untouched rows stay


def test_append_fp8_rejects_slots_past_the_pool():
    k = np.zeros((2, 1, 64), dtype=np.float32)
    kc = np.zeros((2, 1, BLOCK, 64), dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.kv_append_fp8(k, k, np.array([0, 2 * BLOCK]), kc, kc.copy(), 1.0, 1.0)
