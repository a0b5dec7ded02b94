"""Pins for the oracle's row-wise and MX block quantizers (CPU only).

Expected codes in the hand-worked rows are derived here from the E4M3 bit
definition (value = (8+m) * 2^(e-10), subnormals m * 2^-9), not from the
oracle's encoder; the invariants follow from the scale rule amax / 448.
"""

import numpy as np
import pytest

import synth
from oracle import e4m3, quant


def test_power_of_two_scale_row():
    # amax 896 -> s = 896/448 = 2 exactly, so x/s is exact and the codes are
    # those of x/2 in the format table.
    x = np.array([[896.0, 1.0, -3.0, 0.5, 2.0 ** -8, 15 * 2.0 ** -9, -2.0 ** -12, 0.0]], dtype=np.float32)
    q, s = quant.quantize_rowwise(x)
    assert s[0] == 2.0
    # x/2 = 448, 0.5, -1.5, 0.25, 2^-9, 15*2^-10 (tie -> even code 0x08), -2^-13 (-> -0), 0
    assert list(q[0]) == [0x7E, 0x30, 0xBC, 0x28, 0x01, 0x08, 0x80, 0x00]


def test_quotient_rounds_to_fp32_before_the_cast():
    """The quotient is the fp32 x / s (reading P2: a correctly rounded fp32
    divide, then the E4M3 rounding).  These elements make the fp32 quotient
    land exactly on an E4M3 midpoint while the exact quotient lies just off
    it, so a float64 divide would round the other way.

    amax = 448 + 7*2^-14 = 448 (1 + 2^-20), so s = amax / 448 = 1 + 2^-20
    exactly.
      x1 = 1.0625 + 9*2^-23 = 1.0625 s + 2^-24: x1 / s = 1.0625 + 2^-24 / s,
        less than half an fp32 ulp (2^-23 near 1) above 1.0625, so
        fp32(x1 / s) = 1.0625, the midpoint of 1.0 (0x38) and 1.125 (0x39); the
        tie goes to the even mantissa, 0x38.  Exactly, x1 / s > 1.0625: 0x39.
      x2 = 1.1875 + 9*2^-23 = 1.1875 s - 2^-24: fp32(x2 / s) = 1.1875, the
        midpoint of 1.125 (0x39) and 1.25 (0x3A); ties to even: 0x3A.  Exactly,
        x2 / s < 1.1875: 0x39.
    The negated elements take the same codes with the sign bit.
    """
    amax = 448.0 + 7 * 2.0 ** -14
    x1 = 1.0625 + 9 * 2.0 ** -23
    x2 = 1.1875 + 9 * 2.0 ** -23
    x = np.array([[amax, x1, x2, -x1, -x2]], dtype=np.float32)
    assert np.array_equal(x.astype(np.float64), np.array([[amax, x1, x2, -x1, -x2]]))   # all exact in fp32
    q, s = quant.quantize_rowwise(x)
    assert s[0] == np.float32(1 + 2.0 ** -20)
    # the two roundings of each quotient, as worked out above
    assert np.float32(x[0, 1]) / s[0] == np.float32(1.0625) and float(x1) / float(s[0]) > 1.0625
    assert np.float32(x[0, 2]) / s[0] == np.float32(1.1875) and float(x2) / float(s[0]) < 1.1875
    assert list(q[0]) == [0x7E, 0x38, 0x3A, 0xB8, 0xBA]


def test_unit_scale_row_is_plain_cast():
    # amax 448 -> s = 1: the quantizer reduces to the cast itself.
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 300)).astype(np.float32) * 40
    x[:, 0] = 448.0
    q, s = quant.quantize_rowwise(x)
    assert np.all(s == 1.0)
    import torch
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_zero_and_tiny_rows():
    x = np.array([[0.0, -0.0, 0.0, -0.0],
                  [0.0, 0.0, 1e-45, -1e-45],       # amax 2^-149: amax/448 underflows to 0
                  [0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    q, s = quant.quantize_rowwise(x)
    assert np.all(s == 0.0)
    assert list(q[0]) == [0x00, 0x80, 0x00, 0x80]
    assert list(q[1]) == [0x00, 0x00, 0x00, 0x80]
    assert list(q[2]) == [0, 0, 0, 0]


def test_empty_shapes():
    q, s = quant.quantize_rowwise(np.zeros((3, 0), np.float32))
    assert q.shape == (3, 0) and list(s) == [0, 0, 0]
    q, s = quant.quantize_rowwise(np.zeros((0, 5), np.float32))
    assert q.shape == (0, 5) and s.shape == (0,)


def test_single_nonzero_row():
    x = np.zeros((1, 64), np.float32)
    x[0, 17] = -3.25
    q, s = quant.quantize_rowwise(x)
    assert s[0] == np.float32(np.float32(3.25) / np.float32(448))
    assert q[0, 17] == 0xFE and np.all(np.delete(q[0], 17) == 0)


def _rows_of_all_kinds(n_rows=64, cols=257):
    w = synth.WORKLOADS["c4_ffn_up_8192x22016x8192"]
    x = synth.draw(w, "a", slice(0, n_rows))[:, :cols].copy()
    x[1] *= 1e-36                       # subnormal-adjacent scales
    x[2] *= 1e30
    x[3] = np.abs(x[3])
    x[4] = -np.abs(x[4])
    return x


def test_amax_element_maps_to_448():
    x = _rows_of_all_kinds()
    q, s = quant.quantize_rowwise(x)
    normal = s >= np.float32(2.0 ** -126)
    assert normal.sum() >= x.shape[0] - 1
    for r in np.nonzero(normal)[0]:
        j = np.argmax(np.abs(x[r]))
        assert q[r, j] & 0x7F == 0x7E
        assert (q[r, j] >> 7) == np.signbit(x[r, j])


def test_error_bound():
    """|dec(q) s - x| <= (2^-4 + 2^-22)|x| + 2^-10 s for normal s (float64)."""
    x = _rows_of_all_kinds()
    q, s = quant.quantize_rowwise(x)
    d = e4m3.decode(q) * s.astype(np.float64)[:, None]
    err = np.abs(d - x.astype(np.float64))
    bound = (2.0 ** -4 + 2.0 ** -22) * np.abs(x.astype(np.float64)) + 2.0 ** -10 * s[:, None]
    assert np.all(err <= bound)
    # the bound is tight enough to notice a wrong scale or a dropped rounding step
    assert np.max(err / np.maximum(bound, 1e-300)) > 0.3


def test_subnormal_scale_saturates():
    # s = fp32(amax/448) is subnormal and coarse: amax/s exceeds 448 and must saturate.
    t = 2.0 ** -149                                   # smallest fp32 subnormal
    x = np.array([[1075 * t, 300 * t, -1075 * t]], dtype=np.float32)
    q, s = quant.quantize_rowwise(x)
    assert s[0] == np.float32(2 * t)                  # 1075/448 = 2.3996 -> 2 subnormal steps
    assert 0 < s[0] < 2.0 ** -126
    assert np.float32(x[0, 0] / s[0]) > 448.0
    # 300t / 2t = 150 lies between 144 = 9*2^4 (e=14, m=1: 0x71) and 160 = 10*2^4 (0x72); nearer 144
    assert list(q[0]) == [0x7E, 0x71, 0xFE]


# ---------------------------------------------------------------- MX blocks

def test_mx_exponent_against_scan():
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        np.ldexp(448.0, np.arange(-140, 120)),                        # exact powers of two x 448
        np.nextafter(np.ldexp(448.0, np.arange(-120, 110)), np.inf),  # one ulp above them
        np.exp(rng.uniform(-80, 80, 2000)),
        [0.0, 1e-45, 3.4e38],
    ]).astype(np.float32).astype(np.float64)
    e = quant.mx_block_exponent(amax)
    for a, ei in zip(amax, e):
        if a == 0:
            assert ei == -127
            continue
        # brute force: the smallest integer t in [-127, 127] with a <= 448 * 2^t
        want = next(t for t in range(-127, 128) if a <= 448.0 * 2.0 ** t)
        assert ei == want, (a, ei, want)


def test_mx_quantize_blocks():
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    x = synth.draw(w, "a", slice(0, 16))[:, :256]
    q, e = quant.mx_quantize(x)
    assert q.shape == (16, 256) and e.shape == (16, 8) and e.dtype == np.uint8
    blocks = x.reshape(16, 8, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    scaled = amax * np.ldexp(1.0, 127 - e.astype(np.int64))
    assert np.all((scaled > 224) & (scaled <= 448))
    dec = e4m3.decode(q).reshape(16, 8, 32)
    top = np.take_along_axis(np.abs(dec), np.abs(blocks).argmax(axis=2)[:, :, None], 2)[..., 0]
    assert np.all((top >= 224) & (top <= 448))
    # dequantized values stay within the E4M3 half-ulp of the scaled input
    back = dec * quant.ue8m0_value(e)[:, :, None]
    err = np.abs(back - blocks)
    assert np.all(err <= 2.0 ** -4 * np.abs(blocks) + 2.0 ** -10 * quant.ue8m0_value(e)[:, :, None])


def test_mx_zero_block():
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = 1.0
    q, e = quant.mx_quantize(x)
    assert list(e[0]) == [0, 0] and list(e[1]) == [0, 127 - 8]   # 1.0 -> e = -8, 2^8 = 256 in (224, 448]
    assert q[1, 40] == 0x78 and np.count_nonzero(q) == 1           # 256 = (8+0)*2^(15-10)


def test_mx_rejects_ragged_k():
    with pytest.raises(ValueError):
        quant.mx_quantize(np.zeros((1, 33), np.float32))


def test_bf16_to_f32_matches_torch_every_pattern():
    """All 65536 bfloat16 patterns against torch's own bf16 -> fp32 conversion
    (NaN patterns compared as NaN)."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = quant.bf16_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_tensorwise_power_of_two_example():
    # amax 896 over the whole tensor -> s = 2; codes are those of x / 2 in the
    # format table (hand-derived as in test_power_of_two_scale_row)
    x = np.array([[1.0, -3.0, 0.5], [2.0 ** -8, 896.0, -2.0 ** -12]], dtype=np.float32)
    q, s = quant.quantize_tensorwise(x)
    assert s.tolist() == [2.0]
    assert q.tolist() == [[0x30, 0xBC, 0x28], [0x01, 0x7E, 0x80]]


def test_tensorwise_is_rowwise_of_the_flattened_tensor():
    # one scale for all elements = the row-wise rule applied to a single row
    w = synth.Workload("t", 37, 37, 300, "a", "rowfactor_outlier", "normal", "rowwise", 21)
    x = synth.draw(w, "a")
    q, s = quant.quantize_tensorwise(x)
    qr, sr = quant.quantize_rowwise(x.reshape(1, -1))
    assert np.array_equal(q.reshape(1, -1), qr) and np.array_equal(s, sr)


def test_tensorwise_zero_and_empty():
    q, s = quant.quantize_tensorwise(np.array([[0.0, -0.0]], np.float32))
    assert s.tolist() == [0.0] and q.tolist() == [[0x00, 0x80]]
    q, s = quant.quantize_tensorwise(np.zeros((0, 5), np.float32))
    assert s.tolist() == [0.0] and q.shape == (0, 5)


# ---------------------------------------------------------------- E5M2 output
# Expected codes below are worked from the E5M2 bit definition (value =
# (4+m) * 2^(e-17), subnormals m * 2^-16), not from the oracle's encoder.

from oracle import e5m2  # noqa: E402


def test_e5m2_power_of_two_scale_row():
    # amax 114688 -> s = 114688 / 57344 = 2 exactly; codes are those of x / 2
    x = np.array([[114688.0, 1.0, -3.0, 0.5, 2.0 ** -15, 3 * 2.0 ** -16, -2.0 ** -20, 0.0]], dtype=np.float32)
    q, s = quant.quantize_rowwise(x, "e5m2")
    assert s[0] == 2.0
    # x/2 = 57344, 0.5, -1.5, 0.25, 2^-16, 1.5*2^-16 (tie between subnormal codes 1 and 2 -> even),
    # -2^-21 (-> -0), 0
    assert list(q[0]) == [0x7B, 0x38, 0xBE, 0x34, 0x01, 0x02, 0x80, 0x00]


def test_e5m2_unit_scale_row_is_plain_cast():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 300)).astype(np.float32) * 3000
    x[:, 0] = -57344.0
    q, s = quant.quantize_rowwise(x, "e5m2")
    assert np.all(s == 1.0)
    import torch
    assert np.array_equal(q, torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy())


def test_e5m2_amax_element_maps_to_max_and_error_bound():
    x = _rows_of_all_kinds()
    q, s = quant.quantize_rowwise(x, "e5m2")
    normal = s >= np.float32(2.0 ** -126)
    assert normal.sum() >= x.shape[0] - 1
    for r in np.nonzero(normal)[0]:
        j = np.argmax(np.abs(x[r]))
        assert q[r, j] & 0x7F == 0x7B and (q[r, j] >> 7) == np.signbit(x[r, j])
    # |dec(q) s - x| <= (2^-3 + 2^-22)|x| + 2^-17 s: half an E5M2 step (2 mantissa bits), the fp32
    # division, and half the subnormal step
    d = e5m2.decode(q[normal]) * s[normal].astype(np.float64)[:, None]
    xn = x[normal].astype(np.float64)
    bound = (2.0 ** -3 + 2.0 ** -22) * np.abs(xn) + 2.0 ** -17 * s[normal].astype(np.float64)[:, None]
    err = np.abs(d - xn)
    assert np.all(err <= bound) and np.max(err / bound) > 0.3
    # E5M2 keeps less precision than E4M3 on the same rows
    q4, s4 = quant.quantize_rowwise(x[normal])
    err4 = np.abs(e4m3.decode(q4) * s4.astype(np.float64)[:, None] - xn)
    assert err.sum() > err4.sum()


def test_e5m2_tensorwise_is_rowwise_of_the_flattened_tensor():
    w = synth.WORKLOADS["c2_2048x1024x4096"]
    x = synth.draw(w, "a", slice(0, 16))[:, :500].copy()
    q, s = quant.quantize_tensorwise(x, "e5m2")
    q1, s1 = quant.quantize_rowwise(x.reshape(1, -1), "e5m2")
    assert np.array_equal(q.reshape(1, -1), q1) and s[0] == s1[0]
    assert s[0] == np.float32(np.float32(np.abs(x).max()) / np.float32(57344.0))
