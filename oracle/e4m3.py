"""OCP OFP8 e4m3fn codec (test infrastructure only; see the package header).

The pages say only "FP8" (page 2, section 8, "W8A8 Block FP8"); the variant
is the OCP e4m3fn format ("fn" = finite, no infinities), as used by the
DeepSeek-style block-FP8 checkpoints the pages' tuning script targets. The
encoding is defined by the OCP 8-bit floating point specification:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent 0 is subnormal: value = (m / 8) * 2^-6;
* exponents 1..15 are normal: value = (1 + m / 8) * 2^(e - 7);
* exponent 15 with mantissa 7 (codes 0x7F and 0xFF) is NaN; there is no
  infinity, so the largest finite magnitude is 0x7E = 1.75 * 2^8 = 448.

Rounding into e4m3 is round-to-nearest, ties to the even code (mantissa LSB
0), with the sign applied afterwards so that -0 and negative underflow give
0x80. Inputs must already lie in [-448, 448]; the quantisers clamp first.
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_CODES = (0x7F, 0xFF)


def _code_value(code: int) -> float:
    """Value of one e4m3fn code from the OCP closed form, as a Python float."""
    sign = code >> 7
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return -mag if sign else mag


# Decode table for all 256 codes, float64 (every finite value is exact).
_TABLE = np.array([_code_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite codes 0x00..0x7E in increasing order of value, and the
# exact midpoints between neighbours (all exact in float32 and float64).
_POS_VALUES = _TABLE[:0x7F].copy()
_MIDPOINTS = (_POS_VALUES[:-1] + _POS_VALUES[1:]) / 2.0


def e4m3_values() -> np.ndarray:
    """All 256 decoded values (NaN at 0x7F and 0xFF), float64."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 e4m3fn codes to float64 values (NaN codes give NaN)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode_rne(v) -> np.ndarray:
    """Round float32 values in [-448, 448] to e4m3fn codes, nearest-even.

    For each |v| the nearest non-negative finite e4m3 value is found by
    exact comparison with the midpoints between neighbouring codes: below a
    midpoint the lower code wins, above it the upper code; exactly on a
    midpoint the code whose mantissa LSB is 0 wins. The sign bit of v is then
    ORed in, so -0.0 and negatives that round to zero give 0x80.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode_rne: non-finite input")
    mag = np.abs(v).astype(np.float64)
    if np.any(mag > E4M3_MAX):
        raise ValueError("e4m3_encode_rne: |v| > 448; clamp before encoding")
    # lower = the largest code whose value is <= |v|; at 0x7E there is no
    # upper neighbour inside the clamp range.
    lower = np.searchsorted(_POS_VALUES, mag, side="right") - 1
    has_upper = lower < 0x7E
    mid = _MIDPOINTS[np.minimum(lower, 0x7D)]
    above = has_upper & (mag > mid)
    tie = has_upper & (mag == mid)
    take_upper = above | (tie & ((lower & 1) == 1))
    code = np.where(take_upper, lower + 1, lower).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)
