"""Pins of the oracle's number formats against library routines (torch's float8_e4m3fn and bfloat16
casts), run exhaustively where the format is small enough."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    # the format's landmarks: max 448, min normal 2^-6, min subnormal 2^-9, NaN at 0x7F / 0xFF
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))


def _torch_encode(x: np.ndarray) -> np.ndarray:
    """torch's cast rounds to nearest even but does not saturate: clamp to +-448 first."""
    t = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_every_bf16_value_matches_torch():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    finite = np.isfinite(vals)
    vals = vals[finite]
    ref = _torch_encode(vals)
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    # -0.0 and values that round to zero keep their sign in both
    assert np.array_equal(got, ref)


def test_e4m3_encode_fp32_sweep_and_ties_match_torch():
    rng = np.random.default_rng(7)
    sweep = np.concatenate([
        rng.uniform(-500, 500, 20000),
        rng.uniform(-1, 1, 20000),
        np.exp(rng.uniform(-16, 6.2, 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    # exact ties between neighbouring codes (mid-points), both normal and subnormal
    mids = []
    for c in range(0, 0x7E):
        a, b = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mids += [(a + b) / 2, -(a + b) / 2]
    vals = np.concatenate([sweep, np.array(mids, np.float32)])
    ref = _torch_encode(vals)
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,code", [
    (448.0, 0x7E), (449.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (float("inf"), 0x7E),
    (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
])
def test_e4m3_encode_saturation_and_ties(x, code):
    assert oracle.e4m3_encode(x) == code
    assert oracle.e4m3_encode(float("nan")) == 0x7F


def test_bf16_decode_all_values_match_torch():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    for h in range(0, 65536, 1):
        got = oracle.bf16_decode(h)
        r = ref[h]
        assert (math.isnan(got) and math.isnan(r)) or got == r, h
