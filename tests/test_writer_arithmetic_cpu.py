"""The arithmetic the E4M3 bulk writer relies on, checked on the CPU.

The writer stores E4M3(x / scale).  Instead of one IEEE float32 division per
element it uses the reciprocal r = RN(1/scale) and one FMA correction,
q0 = RN(a r), e = RN(a - q0 scale), q = RN(q0 + e r) (Markstein's division
theorem: q is the correctly rounded a / scale when nothing underflows), and
a branch-free encoder: round at the third mantissa bit by adding 0x7FFFF plus
the kept last bit, multiples of 2^-9 below 2^-6, 448 and above saturate, NaN
to 0x7F.  These tests compute both in numpy, with an exact FMA emulation, and
compare them with numpy's IEEE float32 division and the oracle's nearest-code
encoder (which the E4M3 pins tie to the format definition and torch).
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


def branch_free_code(q):
    a = q.view(np.uint32)
    rn = (a + np.uint32(0x7FFFF) + ((a >> np.uint32(20)) & np.uint32(1))).astype(np.uint32)
    normal = ((rn >> np.uint32(20)) - np.uint32(960)).astype(np.uint32)
    with np.errstate(all="ignore"):
        sub = np.rint(q * np.float32(512))
    sub = np.where(a < 0x3C800000, sub, 0).astype(np.uint32)
    c = np.where(a < 0x3C800000, sub, normal)
    c = np.where(a >= 0x43E00000, 0x7E, c)
    return np.where(a > 0x7F800000, 0x7F, c).astype(np.uint8)


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


def test_branch_free_encoder_equals_the_nearest_code_search():
    """Every rounding case of the encoder: each 11-bit prefix (exponent and the
    3 kept mantissa bits) with the remaining 20 bits at 0, 1, just below half,
    exactly half, just above half and all ones, plus every pattern below 2^-6
    on a 2^7 grid and its neighbours (ties of the 2^-9 grid), infinity and
    NaNs."""
    prefix = np.arange(0, 1 << 11, dtype=np.uint32) << np.uint32(20)
    rests = np.array([0, 1, 0x7FFFF, 0x80000, 0x80001, 0xFFFFF], np.uint32)
    a = (prefix[:, None] | rests[None, :]).ravel()
    low = np.arange(0, 0x3C800000, 1 << 7, dtype=np.uint32)
    a = np.concatenate([a, low, low + 1, np.maximum(low, 1) - 1,
                        np.array([0x7F800000, 0x7F800001, 0x7FC00000, 0x7FFFFFFF], np.uint32)])
    a = a[a <= 0x7FFFFFFF]
    q = a.view(np.float32)
    with np.errstate(invalid="ignore"):
        ref = oracle.encode_e4m3(q)
    assert np.array_equal(branch_free_code(q), ref)
