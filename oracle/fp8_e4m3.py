"""OCP 8-bit floating point, E4M3 "fn" variant: a plain codec for the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

The pages say only that the KV writer "supports FP8 KV-cache quantized writes"
(TGI PagedAttention 深度解析, §4.1, the paragraph on the KV write side) and list
FP8 among vLLM's quantisations (10分钟学懂VLLM内部原理, "vLLM优缺点").  Which FP8
and how it rounds is not on the pages; the reading taken here is the OCP E4M3FN
format (the native OCP format of CDNA4), written out from the format definition:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals m * 2^-9, m = 1..7 (and zero);
* exponent field e = 1..15 encodes (1 + m/8) * 2^(e-7);
* the single pattern S.1111.111 is NaN; there is no infinity;
* hence the largest finite magnitude is S.1111.110 = 448.

The quantiser rounds to the nearest representable value, ties to the code with
an even last bit, saturates magnitudes above 448 (infinities included) to 448,
maps NaN to 0x7F with the input's sign bit, and keeps the sign of zero.

This is done by brute force: the 127 non-negative finite code values are
tabulated from the definition above and the nearest one is searched; no bit
tricks are used, so that the code can be checked against the definition by eye.
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_value_of_code(code: int) -> float:
    """Exact value of one 8-bit code, from the format definition (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Values of codes 0x00..0x7E (all non-negative finite codes), ascending.
_POS_VALUES = np.array([e4m3_value_of_code(c) for c in range(0x7F)], dtype=np.float64)
assert np.all(np.diff(_POS_VALUES) > 0)
assert _POS_VALUES[-1] == E4M3_MAX

# Value of every code 0..255 (NaN at 0x7F and 0xFF).
_ALL_VALUES = np.array([e4m3_value_of_code(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes -> exact float64 values (NaN for 0x7F / 0xFF)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _ALL_VALUES[codes]


def encode_e4m3(y) -> np.ndarray:
    """float32 values -> uint8 E4M3FN codes (nearest, ties to even, saturating).

    `y` must already be the float32 value to be stored (the caller performs any
    division by a scale in float32 first).
    """
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    a = np.abs(flat.astype(np.float64))          # exact: float32 -> float64
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))   # saturate (inf -> 448)
    # Nearest of the tabulated values: candidates just below and just above.
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # On a tie, take the candidate whose code is even.
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(flat).astype(np.uint8) << 7
    code = np.where(nan, np.uint8(NAN_CODE), code).astype(np.uint8) | sign
    return code.reshape(y.shape)


def quantize_e4m3(x_f32, scale: float) -> np.ndarray:
    """Store x/scale as E4M3FN: the division is one correctly rounded float32 divide."""
    x32 = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = x32 / np.float32(scale)                # IEEE float32 division
    return encode_e4m3(q.astype(np.float32))
