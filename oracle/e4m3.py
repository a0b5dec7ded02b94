"""OCP E4M3FN ("float8_e4m3fn") in plain Python/numpy -- oracle, test infrastructure.

Source of the format: the pages cast fp32 tensors with
``x.to(torch.float8_e4m3fn)`` (page "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM",
the DeepGEMM GEMM-call example) and state that the largest E4M3 magnitude is
448 (same page, ``_calibrate_scales`` of the hybrid-inference class).  448 is
the largest finite value only in the OCP "FN" variant: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, and a single NaN pattern per
sign (S.1111.111).  (An IEEE-style E4M3 with infinities, or the FNUZ variant
with bias 8, would top out at 240.)

Bit layout of a code c (8 bits): s = c>>7, e = (c>>3)&15, m = c&7.
  * e == 15 and m == 7          -> NaN
  * e == 0                      -> (-1)^s * m * 2^-9          (subnormal)
  * otherwise                   -> (-1)^s * (8 + m) * 2^(e-10) (normal)

The cast fp32 -> E4M3 used by this library (the pages leave rounding and
overflow open; see the readings in the design notes):
  * round to the nearest representable value; a tie goes to the code whose
    mantissa LSB is 0 (round-half-to-even);
  * magnitudes above 448 saturate to 448 (the pages report NaN outputs as the
    failure to avoid: page on FP8 7B inference on an RTX 4060, section 4.1);
  * the sign bit is copied from the input, so tiny negatives give -0 (0x80);
  * NaN input gives 0x7F with the input's sign (outside the contract).
"""

import numpy as np

NAN_CODE = 0x7F
MAX_CODE = 0x7E          # +448
MAX_VALUE = 448.0


def decode_code(c: int) -> float:
    """Value of one E4M3FN code, straight from its bit fields (exact)."""
    if not 0 <= c <= 255:
        raise ValueError("E4M3 code out of range: %r" % (c,))
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = (8 + m) * 2.0 ** (e - 10)
    return -mag if s else mag


# float64 value of every code; NaN at 0x7F and 0xFF.  Every finite entry is an
# integer multiple of 2^-9, so it is exact in float64 (and in float32).
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# The 127 non-negative finite magnitudes in code order 0x00..0x7E.  The format
# is monotone in the code, so this list is sorted ascending.
_MAGS = DECODE_TABLE[:0x7F].copy()


def decode(codes) -> np.ndarray:
    """Decode an array of E4M3FN codes (uint8) to float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


def encode(x) -> np.ndarray:
    """Cast real values to E4M3FN codes: nearest, ties to even, saturating.

    The input is float32 (the cast the pages apply to fp32 tensors); float64
    input is accepted for values that are exact scalings of float32 ones (the
    MX block quantizer).  For each |x| find the two neighbouring magnitudes
    lo <= |x| <= hi in the table, compare |x| with their midpoint (exact in
    float64), and on a tie keep the even code.  Above 448 the result is 448.
    """
    x = np.asarray(x)
    if x.dtype != np.float64:
        x = x.astype(np.float32)
    a = np.abs(x).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    lo = np.searchsorted(_MAGS, a, side="right") - 1      # largest i: mags[i] <= a
    lo = np.clip(lo, 0, MAX_CODE)
    hi = np.minimum(lo + 1, MAX_CODE)
    mid = (_MAGS[lo] + _MAGS[hi]) * 0.5
    go_up = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(go_up, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(NAN_CODE), code).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def is_finite_code(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes & 0x7F) != NAN_CODE
