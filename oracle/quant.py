"""Quantizers in plain numpy -- oracle, test infrastructure.

``quantize_rowwise``: one fp32 scale per row (per token for activations, per
output channel for weights), computed as the row's largest magnitude over 448,
the E4M3 maximum.  Sources: the scale rule ``abs_max / 448.0`` in
``_calibrate_scales`` of the hybrid-inference class on the page
"FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM" (there per tensor; here per row,
as the per-token ``scale_a[m]`` and per-channel ``scale_b[n]`` of the same
page's DeepGEMM call require); the flow "fp32 activation -> statistics ->
dynamic-range calibration -> FP8" in section 2.2 of the page on FP8 7B
inference on an RTX 4060, and its per-token adaptation idea in section 5.

Readings taken where the pages are silent (listed in the design notes):
  * the scale is a dequantization multiplier: x ~ dec(q) * s;
  * s = fp32(amax / 448) with one IEEE round-to-nearest division;
  * q = cast(fp32(x / s)): a correctly rounded fp32 division, then the
    saturating round-to-nearest-even E4M3 cast (two roundings, in this order);
  * if s == 0 (all-zero or empty row, or amax so tiny that amax/448
    underflows), s is written as 0 and every code is a zero with x's sign.

E5M2 output (``fmt="e5m2"``): the same rule with that format's largest
finite value, 57344, in place of 448, and the saturating round-to-nearest-even
E5M2 cast (oracle.e5m2).  The pages take E5M2 beside E4M3 (page on
FlashInfer's concat_mla_k with FP8 inputs, sections 1-2) but state no scale
rule for it; this is the plainest reading of the E4M3 rule for it.

``mx_quantize``: the MXFP8 block quantizer that builds mode-(b) inputs.  One
unsigned 8-bit power-of-two scale per 32 consecutive K elements of each row
(scale tensor shape ``(n, k // 32)`` and ``num_elts_per_sf=32`` on the page
"[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합", section 1, weight
preprocessing).  The scale code c stands for 2^(c-127) (UE8M0); the block
exponent is the smallest e with amax <= 448 * 2^e, i.e. 2^ceil(log2(amax/448)),
clamped to [-127, 127]; an all-zero block takes e = -127.
"""

import numpy as np

from . import e4m3, e5m2

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
_FORMATS = {"e4m3": (e4m3, E4M3_MAX), "e5m2": (e5m2, E5M2_MAX)}
MX_BLOCK = 32
UE8M0_BIAS = 127


def row_scales(x, fmt="e4m3") -> np.ndarray:
    """s[r] = fp32(max_c |x[r,c]| / MAX) (MAX = 448 for E4M3, 57344 for E5M2);
    empty rows give 0."""
    x = np.asarray(x, dtype=np.float32)
    if x.shape[1] == 0:
        return np.zeros(x.shape[0], dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)               # exact: a max does not round
    return (amax / np.float32(_FORMATS[fmt][1])).astype(np.float32)


def quantize_rowwise(x, fmt="e4m3"):
    """Per-row quantization to E4M3 (or E5M2): returns (codes uint8 [R,C], scales fp32 [R])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize_rowwise expects a 2-D array")
    s = row_scales(x, fmt)
    zero_row = s == 0
    safe = np.where(zero_row, np.float32(1.0), s).astype(np.float32)
    y = (x / safe[:, None]).astype(np.float32)     # IEEE fp32 divide, round to nearest
    y = np.where(zero_row[:, None], np.copysign(np.float32(0.0), x), y).astype(np.float32)
    return _FORMATS[fmt][0].encode(y), s


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float32: bf16 is the top half of an
    fp32, so the value converts exactly by shifting its bits up by 16."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_tensorwise(x, fmt="e4m3"):
    """Per-tensor quantization: one scale for the whole tensor, the amax/448 of
    `_calibrate_scales` on the DeepGEMM page (abs_max over the data; amax/57344
    for E5M2).  Returns (codes uint8 [same shape], scale fp32 [1])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    s = np.float32(amax / np.float32(_FORMATS[fmt][1]))       # IEEE fp32 divide
    if s == 0:
        y = np.copysign(np.float32(0.0), x).astype(np.float32)
    else:
        y = (x / s).astype(np.float32)                        # IEEE fp32 divide, round to nearest
    return _FORMATS[fmt][0].encode(y), np.array([s], dtype=np.float32)


def mx_block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127].

    Written as a search from below with exact float64 comparisons (448 * 2^e
    is exact), not with a logarithm, which can misround at powers of two.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                      # a = f * 2^ex, 0.5 <= f < 1
    e = ex.astype(np.int64) - 10             # 448 * 2^(ex-10) < 0.5 * 2^ex <= a
    for _ in range(4):
        e = np.where(a > np.ldexp(E4M3_MAX, e), e + 1, e)
    e = np.where(a == 0, -UE8M0_BIAS, e)
    return np.clip(e, -UE8M0_BIAS, UE8M0_BIAS)


def mx_quantize(x):
    """MXFP8 block quantization along the last axis.

    Returns (codes uint8 [R,C], scale codes uint8 [R, C/32]).  Each block is
    scaled by 2^-e exactly (a power of two) and then cast to E4M3; by the
    choice of e no element exceeds 448, so the cast never saturates.
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("MX blocks need the row length to be a multiple of 32")
    blocks = x.reshape(R, C // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=2)
    e = mx_block_exponent(amax)
    y = np.ldexp(blocks, -e[:, :, None])           # exact power-of-two scaling
    codes = e4m3.encode(y).reshape(R, C)
    return codes, (e + UE8M0_BIAS).astype(np.uint8)


def ue8m0_value(codes) -> np.ndarray:
    """float64 value 2^(c-127) of UE8M0 scale codes (code 255, NaN, is not used)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.ldexp(1.0, c - UE8M0_BIAS)
