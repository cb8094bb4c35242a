"""Pins for the oracle's element decoders (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle.codecs import bf16_to_f64, e4m3fn_to_f64, decode
from workloads import _to_fp8, _to_bf16_bits


# OCP 8-bit floating point spec, e4m3 ("FN") column: selected codes.
E4M3_KNOWN = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
    0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0,
    0xFE: -448.0, 0x81: -(2.0 ** -9),
}


def test_e4m3_known_values():
    for code, val in E4M3_KNOWN.items():
        got = e4m3fn_to_f64(np.array([code], np.uint8))[0]
        assert got == val, (hex(code), got, val)
    nan = e4m3fn_to_f64(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(nan).all()
    neg_zero = e4m3fn_to_f64(np.array([0x80], np.uint8))[0]
    assert neg_zero == 0.0 and math.copysign(1.0, neg_zero) < 0


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert (both_nan | (ours == ref)).all()
    assert int(np.isnan(ours).sum()) == 2


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 20000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = bf16_to_f64(bits)
    ok = (np.isnan(ref) & np.isnan(ours)) | (ref == ours)
    assert ok.all()
    assert bf16_to_f64(np.array([0x3F80, 0xC000, 0x7F80], np.uint16)).tolist() == [1.0, -2.0, math.inf]


def test_scale_applies_as_product():
    codes = np.array([0x38, 0x40, 0xB8], np.uint8)          # 1, 2, -1
    assert decode(codes, "fp8", 0.5).tolist() == [0.5, 1.0, -0.5]


def test_input_quantizer_saturates_and_rounds():
    # The generator's fp8 path: scale = amax/448, clamp, round to nearest.
    x = np.array([1000.0, -3.0, 0.001, 2.5, -1000.0], np.float32)
    codes, scale = _to_fp8(x)
    assert scale == pytest.approx(1000.0 / 448.0, rel=1e-7)
    vals = e4m3fn_to_f64(codes)
    assert not np.isnan(vals).any()
    assert vals[0] == 448.0 and vals[-1] == -448.0
    # every non-saturated value is within half a step of e4m3 (3 mantissa bits)
    rel = np.abs(vals[1:4] * scale - x[1:4]) / np.abs(x[1:4])
    assert (rel[:1] <= 2.0 ** -4).all()
    b = _to_bf16_bits(np.array([1.0, 1.00390625, 1.01171875], np.float32))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 and rounds to even (1.0)
    assert bf16_to_f64(b).tolist() == [1.0, 1.0, 1.015625]
