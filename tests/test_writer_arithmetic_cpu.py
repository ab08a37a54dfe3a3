"""The division the E4M3 bulk writer relies on, checked on the CPU.

The writer stores E4M3(x / scale).  Instead of one IEEE float32 division per
element it uses the reciprocal r = RN(1/scale) and one FMA correction,
q0 = RN(a r), e = RN(a - q0 scale), q = RN(q0 + e r) (Markstein's division
theorem: q is the correctly rounded a / scale when nothing underflows).  This
test computes that sequence in numpy, with an exact FMA emulation, and
compares it with numpy's IEEE float32 division, directly and through the
oracle's nearest-code encoder (which the E4M3 pins tie to the format
definition and torch).
"""
import numpy as np
import pytest

import oracle


def _rn32_of_pair(hi, lo):
    """RN32 of the exact value hi + lo given as a float64 pair (hi = RN64 of
    the sum): rounding hi to float32 is exact unless hi is a float32 midpoint,
    where the sign of lo decides."""
    r = hi.astype(np.float32)
    r64 = r.astype(np.float64)
    toward = np.where(hi > r64, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    nxt = np.nextafter(r, toward)
    mid = (r64 + nxt.astype(np.float64)) / 2
    at_mid = (hi == mid) & (lo != 0) & (hi != r64)
    away = at_mid & (((lo > 0) & (nxt > r)) | ((lo < 0) & (nxt < r)))
    return np.where(away, nxt, r).astype(np.float32)


def fma32(x, y, z):
    """float32 fused multiply-add, exactly: x*y is exact in float64, the sum is
    split into hi + lo by Knuth's two-sum, then rounded once to float32."""
    p = x.astype(np.float64) * y.astype(np.float64)
    z = z.astype(np.float64)
    s = p + z
    bb = s - p
    err = (p - (s - bb)) + (z - bb)
    return _rn32_of_pair(s, err)


def quotient(a, s):
    s = np.float32(s)
    r = np.float32(1) / s
    q0 = (a * r).astype(np.float32)
    e = fma32(-q0, np.full_like(a, s), a)
    return fma32(e, np.full_like(a, r), q0)


def all_16bit_magnitudes():
    u = np.arange(0, 0x8000, dtype=np.uint32)
    f16 = u.astype(np.uint16).view(np.float16).astype(np.float32)
    bf16 = (u << 16).view(np.float32)
    v = np.concatenate([f16, bf16])
    return np.unique(v[np.isfinite(v)])


SCALES = [1.0, 6.0 / 448.0, 1.0 / 32.0, 0.002, 0.011, 0.013, 1.0 / 3.0, 0.37, 7.3,
          1.0000001, 0.99999994, 2.0 ** -59, 2.0 ** 58] + \
    list(np.exp(np.random.default_rng(0).uniform(np.log(2.0 ** -60), np.log(2.0 ** 60), 40)))


@pytest.mark.parametrize("s", SCALES)
def test_reciprocal_quotient_gives_the_codes_of_ieee_division(s):
    """Every finite 16-bit magnitude (up to the saturation cut 1024 s): the
    quotient's E4M3 code equals the code of the IEEE float32 quotient, and
    the quotients themselves are equal wherever they reach 2^-11 (below it
    every code is 0, and for the smallest scales the correction step may
    underflow there)."""
    s = np.float32(s)
    vals = all_16bit_magnitudes()
    a = vals[vals <= np.float32(1024) * s]
    ref = (a / s).astype(np.float32)
    got = quotient(a, s)
    big = ref >= np.float32(2.0 ** -11)
    assert np.array_equal(ref[big].view(np.uint32), got[big].view(np.uint32))
    assert np.array_equal(oracle.encode_e4m3(ref), oracle.encode_e4m3(got))
    # above the cut the true quotient exceeds 448: saturation is right there
    assert (vals[vals > np.float32(1024) * s] / s >= 448).all()
