"""OCP E5M2 ("float8_e5m2") in plain Python/numpy -- oracle, test infrastructure.

Source of the format: the page on FlashInfer's concat_mla_k with FP8 inputs
(sections 1-2) names FP8 E5M2 beside E4M3 as an element type the kernels
take; the pages give no bit layout.  Reading: the OCP 8-bit format E5M2, the
one torch calls float8_e5m2 -- 1 sign bit, 5 exponent bits with bias 15,
2 mantissa bits, with infinities and NaNs as in IEEE 754 binary formats.

Bit layout of a code c (8 bits): s = c>>7, e = (c>>2)&31, m = c&3.
  * e == 31 and m == 0          -> (-1)^s * infinity
  * e == 31 and m != 0          -> NaN
  * e == 0                      -> (-1)^s * m * 2^-16          (subnormal)
  * otherwise                   -> (-1)^s * (4 + m) * 2^(e-17) (normal)
Largest finite magnitude: code 0x7B = 1.75 * 2^15 = 57344.

The cast below serves test-input generation (values to E5M2 codes): nearest,
ties to the even code, magnitudes above 57344 saturate to 57344 (the same
saturating reading as the E4M3 cast), sign copied, NaN to 0x7F with the sign.
"""

import numpy as np

INF_CODE = 0x7C
MAX_CODE = 0x7B          # +57344
MAX_VALUE = 57344.0


def decode_code(c: int) -> float:
    """Value of one E5M2 code, straight from its bit fields (exact)."""
    if not 0 <= c <= 255:
        raise ValueError("E5M2 code out of range: %r" % (c,))
    s = (c >> 7) & 1
    e = (c >> 2) & 0x1F
    m = c & 0x3
    if e == 0x1F:
        mag = float("inf") if m == 0 else float("nan")
    elif e == 0:
        mag = m * 2.0 ** -16
    else:
        mag = (4 + m) * 2.0 ** (e - 17)
    return -mag if s else mag


# float64 value of every code.  Every finite entry is an integer multiple of
# 2^-16 below 2^16, so it is exact in float64 (and in float32).
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# The 124 non-negative finite magnitudes in code order 0x00..0x7B (ascending:
# the format is monotone in the code).
_MAGS = DECODE_TABLE[:MAX_CODE + 1].copy()


def decode(codes) -> np.ndarray:
    """Decode an array of E5M2 codes (uint8) to float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


def encode(x) -> np.ndarray:
    """Cast real values to E5M2 codes: nearest, ties to even, saturating.

    For each |x| take the neighbouring magnitudes lo <= |x| <= hi in the
    table, compare |x| with their midpoint (exact in float64) and on a tie
    keep the code with an even mantissa; above 57344 the result is 57344.
    """
    x = np.asarray(x)
    if x.dtype != np.float64:
        x = x.astype(np.float32)
    a = np.abs(x).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    lo = np.searchsorted(_MAGS, a, side="right") - 1
    lo = np.clip(lo, 0, MAX_CODE)
    hi = np.minimum(lo + 1, MAX_CODE)
    mid = (_MAGS[lo] + _MAGS[hi]) * 0.5
    go_up = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(go_up, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def is_finite_code(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes & 0x7C) != 0x7C
