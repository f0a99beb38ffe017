"""Pins of the oracle's element decoders and its fp8 encoder.

fp16 / bf16 / fp8 decoding is checked code by code against numpy's and
torch's own conversions (library routines), fp8 additionally against values
fixed by the OCP E4M3FN format definition. The encoder (round to nearest
even after clamping to +-448) is checked exhaustively over every fp16 and
bf16 input against torch's cast of the clamped value."""
import math

import numpy as np
import torch

import oracle


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_f16_decode_all_codes():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    for c in range(65536):
        assert _same(oracle.f16_to_double(c), float(ref[c])), hex(c)


def test_bf16_decode_all_codes():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ref = bits.to(torch.float64).numpy()
    for c in range(65536):
        assert _same(oracle.bf16_to_double(c), float(ref[c])), hex(c)


def test_fp8_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.fp8_e4m3_to_double(c), float(ref[c])), hex(c)


def test_fp8_decode_format_points():
    # Values fixed by the E4M3FN definition (bias 7, 3 mantissa bits).
    assert oracle.fp8_e4m3_to_double(0x38) == 1.0
    assert oracle.fp8_e4m3_to_double(0x7E) == 448.0
    assert oracle.fp8_e4m3_to_double(0xFE) == -448.0
    assert oracle.fp8_e4m3_to_double(0x01) == 2.0 ** -9       # smallest subnormal
    assert oracle.fp8_e4m3_to_double(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert oracle.fp8_e4m3_to_double(0x08) == 2.0 ** -6       # smallest normal
    assert oracle.fp8_e4m3_to_double(0x77) == 240.0           # exponent 14, mantissa 7
    assert oracle.fp8_e4m3_to_double(0x78) == 256.0           # exponent 15 is finite
    assert math.isnan(oracle.fp8_e4m3_to_double(0x7F))
    assert math.isnan(oracle.fp8_e4m3_to_double(0xFF))
    assert oracle.fp8_e4m3_to_double(0x80) == 0.0 and math.copysign(1, oracle.fp8_e4m3_to_double(0x80)) < 0
    finite = [c for c in range(256) if not math.isnan(oracle.fp8_e4m3_to_double(c))]
    assert len(finite) == 254


def test_fp8_encode_points():
    assert oracle.fp8_e4m3_encode(1.0) == 0x38
    assert oracle.fp8_e4m3_encode(1.0625) == 0x38    # tie between 1.0 and 1.125 -> even
    assert oracle.fp8_e4m3_encode(1.1875) == 0x3A    # tie between 1.125 and 1.25 -> even
    assert oracle.fp8_e4m3_encode(1000.0) == 0x7E    # saturates at 448
    assert oracle.fp8_e4m3_encode(-1000.0) == 0xFE
    assert oracle.fp8_e4m3_encode(2.0 ** -10) == 0x00   # tie between 0 and 2^-9 -> even (0)
    assert oracle.fp8_e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 ulps -> 2
    assert oracle.fp8_e4m3_encode(3.0, 2.0) == oracle.fp8_e4m3_encode(1.5)
    assert oracle.fp8_e4m3_encode(float("nan")) == 0x7F


def _encode_exhaustive(values: np.ndarray):
    x = torch.from_numpy(values.astype(np.float32))
    ref = torch.clamp(x, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, val in enumerate(values):
        if np.isnan(val):
            continue
        got = oracle.fp8_e4m3_encode(float(val))
        assert got == ref[i], (float(val), hex(got), hex(ref[i]))


def test_fp8_encode_all_fp16_inputs():
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = vals[np.isfinite(vals)]
    _encode_exhaustive(vals.astype(np.float64))


def test_fp8_encode_all_bf16_inputs():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    vals = bits.to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    _encode_exhaustive(vals)
