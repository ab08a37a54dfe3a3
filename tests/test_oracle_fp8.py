"""Pins of the oracle's E4M3FN codec (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import decode_e4m3, encode_e4m3, quantize_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def _parse_value(tok):
    if tok == "nan":
        return float("nan")
    if tok == "-nan":
        return math.copysign(float("nan"), -1.0)
    return float(tok)


def _golden():
    dec, enc = [], []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "decode":
                dec.append((int(line[1], 16), _parse_value(line[2])))
            else:
                enc.append((_parse_value(line[1]), int(line[2], 16)))
    return dec, enc


def test_golden_decode_values():
    dec, _ = _golden()
    assert len(dec) >= 10
    for code, val in dec:
        got = float(decode_e4m3(np.array([code], np.uint8))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_golden_encode_values():
    _, enc = _golden()
    assert len(enc) >= 10
    for val, code in enc:
        got = int(encode_e4m3(np.array([val], np.float32))[0])
        assert got == code, (val, hex(got), hex(code))


def test_roundtrip_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    back = encode_e4m3(vals[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])


def test_monotone_and_symmetric():
    pos = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(-pos, neg)


@pytest.mark.parametrize("scale", [1.0, 6.0 / 448.0, 1.0 / 32.0, 0.002])
def test_matches_torch_saturating_cast_on_all_bf16(scale):
    """Library routine: torch's float8_e4m3fn cast (round to nearest even) after an
    explicit clamp to +-448 gives the same code for every bf16 bit pattern."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x32 = bits.to(torch.float32)
    y = x32 / torch.tensor(scale, dtype=torch.float32)
    ref = torch.clamp(y, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = quantize_e4m3(x32.numpy(), scale)
    assert np.array_equal(got, ref)


def test_saturation_and_nan_sign():
    x = np.array([np.inf, -np.inf, 1e30, -1e30, np.nan, -np.nan], np.float32)
    x[5] = np.copysign(np.float32(np.nan), np.float32(-1))
    got = encode_e4m3(x).tolist()
    assert got == [0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0xFF]


def test_quantize_divides_with_one_float32_rounding():
    """x / scale is one correctly rounded float32 quotient.  For float32 operands a
    float64 quotient rounded once to float32 is the correctly rounded result (float64
    carries more than 2*24+2 bits), which gives an independent expected value."""
    rng = np.random.default_rng(7)
    xs = rng.standard_normal(20000).astype(np.float32) * np.float32(4)
    for s in (0.3, 6.0 / 448.0, 1.0 / 7.0):
        s32 = np.float32(s)
        q = (xs.astype(np.float64) / np.float64(s32)).astype(np.float32)
        assert np.array_equal(quantize_e4m3(xs, s), encode_e4m3(q))
