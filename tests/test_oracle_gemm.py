"""Pins for the oracle's two GEMM definitions and its error bound (CPU only).

  * exact rational brute force (fractions.Fraction, pure-Python loops) on tiny
    shapes, for both modes;
  * an integer cross-check: decoded values times 2^9 are integers, so the
    mode-(a) sum times 2^18 must equal an int64 matmul bit for bit;
  * closed forms: all-ones operands, one-hot (permutation) B, and the full
    product table of every pair of finite codes against torch's decode;
  * mode (b) special cases that reduce to mode (a), and the association of
    each scale byte with its 32-element block;
  * the bf16/fp32 ulp used by the bound, at known points.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, gemm, quant


def _codes(seed, shape):
    return synth.u8_codes(seed, 1, shape)


def _frac_dec(c):
    return Fraction(e4m3.decode_code(int(c)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 2, 48), (3, 3, 33)])
def test_mode_a_rational_brute_force(M, N, K):
    A = _codes(100 + K, (M, K))
    B = _codes(200 + K, (N, K))
    sa = synth.scales(synth.WORKLOADS["c1_128x256x512"], "a")[:M]
    sb = synth.scales(synth.WORKLOADS["c1_128x256x512"], "b")[:N]
    D = gemm.gemm_scaled(A, B, sa, sb)
    for m in range(M):
        for n in range(N):
            s = sum(_frac_dec(A[m, k]) * _frac_dec(B[n, k]) for k in range(K))
            exact = s * Fraction(float(sa[m])) * Fraction(float(sb[n]))
            # two float64 roundings after an exact sum
            assert abs(Fraction(D[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 51)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 2, 96)])
def test_mode_b_rational_brute_force(M, N, K):
    A = _codes(300 + K, (M, K))
    B = _codes(400 + K, (N, K))
    ea = synth.u8_codes(5, 2, (M, K // 32)) % 40 + 107
    eb = synth.u8_codes(6, 3, (N, K // 32)) % 40 + 107
    D = gemm.mxfp8_gemm(A, B, ea, eb)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            for k in range(K):
                j = k // 32
                scale = Fraction(2) ** (int(ea[m, j]) - 127) * Fraction(2) ** (int(eb[n, j]) - 127)
                exact += scale * _frac_dec(A[m, k]) * _frac_dec(B[n, k])
            assert abs(Fraction(D[m, n]) - exact) <= (K // 32) * Fraction(1, 2 ** 52) * \
                sum(abs(_frac_dec(A[m, k]) * _frac_dec(B[n, k])) * Fraction(2) ** (int(ea[m, k // 32]) + int(eb[n, k // 32]) - 254)
                    for k in range(K)) + Fraction(1, 2 ** 1000)


def test_mode_a_integer_crosscheck():
    M, N, K = 37, 29, 1000
    A = _codes(11, (M, K))
    B = _codes(12, (N, K))
    # integer image of each code: dec * 2^9 (exact integers, from torch's decode)
    ia = (torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float64) * 512).to(torch.int64)
    ib = (torch.from_numpy(B).view(torch.float8_e4m3fn).to(torch.float64) * 512).to(torch.int64)
    S_int = (ia @ ib.T).numpy()
    ones = np.ones(M, np.float32), np.ones(N, np.float32)
    S = gemm.gemm_scaled(A, B, *ones)
    assert np.array_equal(S * 2.0 ** 18, S_int.astype(np.float64))
    assert np.all(np.abs(S_int) < 2 ** 53)


def test_all_ones_closed_form():
    M, N, K = 5, 7, 8192
    A = np.full((M, K), 0x38, np.uint8)          # 1.0
    B = np.full((N, K), 0x38, np.uint8)
    sa = np.linspace(0.5, 2, M).astype(np.float32)
    sb = np.linspace(2, 0.5, N).astype(np.float32)
    D = gemm.gemm_scaled(A, B, sa, sb)
    assert np.array_equal(D, 8192.0 * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :])


def test_one_hot_b_picks_columns_of_a():
    M, N, K = 6, 9, 64
    A = _codes(21, (M, K))
    perm = (np.arange(N) * 7 + 3) % K
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), perm] = 0x38
    sa = np.arange(1, M + 1, dtype=np.float32)
    sb = np.full(N, 0.5, np.float32)
    D = gemm.gemm_scaled(A, B, sa, sb)
    dec_a = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = dec_a[:, perm] * sa[:, None] * 0.5
    assert np.array_equal(D, want)


def test_product_table_every_code_pair():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    K = 64
    A = np.zeros((finite.size, K), np.uint8)
    B = np.zeros((finite.size, K), np.uint8)
    A[:, 0] = finite
    B[:, 0] = finite
    D = gemm.gemm_scaled(A, B, np.ones(finite.size, np.float32), np.ones(finite.size, np.float32))
    dec = torch.from_numpy(finite).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(D, np.outer(dec, dec))


def test_mode_b_neutral_scales_equal_mode_a():
    M, N, K = 8, 12, 256
    A, B = _codes(31, (M, K)), _codes(32, (N, K))
    ea = np.full((M, K // 32), 127, np.uint8)
    eb = np.full((N, K // 32), 127, np.uint8)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    assert np.array_equal(gemm.mxfp8_gemm(A, B, ea, eb), gemm.gemm_scaled(A, B, ones_m, ones_n))


def test_mode_b_row_constant_scales_equal_mode_a():
    M, N, K = 8, 12, 256
    A, B = _codes(33, (M, K)), _codes(34, (N, K))
    alpha = (np.arange(M) * 5 % 23 + 115).astype(np.uint8)
    beta = (np.arange(N) * 3 % 19 + 118).astype(np.uint8)
    ea = np.repeat(alpha[:, None], K // 32, axis=1)
    eb = np.repeat(beta[:, None], K // 32, axis=1)
    sa = np.ldexp(1.0, alpha.astype(np.int64) - 127).astype(np.float32)
    sb = np.ldexp(1.0, beta.astype(np.int64) - 127).astype(np.float32)
    assert np.array_equal(gemm.mxfp8_gemm(A, B, ea, eb), gemm.gemm_scaled(A, B, sa, sb))


def test_mode_b_scale_association():
    """Only block j is nonzero, with one product: D = 2^(ea+eb-254) dec(a) dec(b)."""
    K = 128
    for j in range(K // 32):
        for t in (0, 31):
            A = np.zeros((3, K), np.uint8)
            B = np.zeros((2, K), np.uint8)
            A[:, 32 * j + t] = [0x38, 0x7E, 0x81]
            B[:, 32 * j + t] = [0x40, 0xB9]
            ea = np.full((3, 4), 127, np.uint8)
            eb = np.full((2, 4), 127, np.uint8)
            ea[:, j] = [100, 150, 127]
            eb[:, j] = [130, 90]
            D = gemm.mxfp8_gemm(A, B, ea, eb)
            da = np.array([1.0, 448.0, -2.0 ** -9])
            db = np.array([2.0, -1.125])
            sa = np.ldexp(1.0, np.array([100, 150, 127]) - 127)
            sb = np.ldexp(1.0, np.array([130, 90]) - 127)
            assert np.array_equal(D, np.outer(da * sa, db * sb))


def test_mx_quantized_gemm_tracks_fp32_product():
    """Quantize fp32 operands with the MX rule; the MX GEMM stays near the
    float64 product of the unquantized inputs (sanity, not a tight pin)."""
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    xa = synth.draw(w, "a", slice(0, 8))[:, :512]
    xb = synth.draw(w, "b", slice(0, 8))[:, :512]
    qa, ea = quant.mx_quantize(xa)
    qb, eb = quant.mx_quantize(xb)
    D = gemm.mxfp8_gemm(qa, qb, ea, eb)
    ref = xa.astype(np.float64) @ xb.astype(np.float64).T
    W = np.abs(xa).astype(np.float64) @ np.abs(xb).astype(np.float64).T
    assert np.all(np.abs(D - ref) <= 0.13 * W)


def test_ulp_values():
    x = np.array([1.0, 1.5, 2.0 ** -130, 0.0, -3.0, 2.0 ** 20 - 1, 2.0 ** -126])
    assert list(gemm.ulp(x, "bf16")) == [2.0 ** -7, 2.0 ** -7, 2.0 ** -133, 2.0 ** -133,
                                         2.0 ** -6, 2.0 ** 12, 2.0 ** -133]
    assert list(gemm.ulp(x, "f32")) == [2.0 ** -23, 2.0 ** -23, 2.0 ** -149, 2.0 ** -149,
                                        2.0 ** -22, 2.0 ** -4, 2.0 ** -149]
    # just below a power of two (log2 can round up there)
    y = np.nextafter(np.ldexp(1.0, np.arange(-100, 100)), 0)
    assert np.array_equal(gemm.ulp(y, "bf16"), np.ldexp(1.0, np.arange(-101, 99) - 7).clip(2.0 ** -133))


def test_check_accepts_bf16_rounding_and_rejects_errors():
    M, N, K = 16, 16, 512
    A, B = _codes(41, (M, K)), _codes(42, (N, K))
    sa = np.ones(M, np.float32)
    sb = np.ones(N, np.float32)
    D = gemm.gemm_scaled(A, B, sa, sb)
    W = gemm.gemm_scaled_weight(A, B, sa, sb)
    bf16 = torch.from_numpy(D).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    ok, ratio, nbad = gemm.check(bf16, D, W, "bf16")
    assert ok and nbad == 0
    wrong = bf16.copy()
    wrong[3, 4] = -wrong[3, 4] + 1.0
    assert not gemm.check(wrong, D, W, "bf16")[0]
    transposed = gemm.gemm_scaled(A, B, sa, sb).T.copy()
    assert not gemm.check(transposed, D, W, "bf16")[0]
    nan = bf16.copy()
    nan[0, 0] = np.nan
    assert not gemm.check(nan, D, W, "bf16")[0]


# ------------------------------------------------- matrix-core alignment term

def _emulate_group_alignment(a_codes, b_codes):
    """Pure-Python model of the in-group alignment described in oracle.gemm:
    per run of 8 K values, products truncated toward zero to a multiple of
    2^(E - 13), E the largest exponent sum of the run (exact rationals)."""
    total = Fraction(0)
    K = len(a_codes)
    for g in range(0, K, 8):
        ks = range(g, min(g + 8, K))
        E = max(int(gemm.code_exponent(a_codes[k])) + int(gemm.code_exponent(b_codes[k])) for k in ks)
        lsb = Fraction(2) ** (E - 13)
        for k in ks:
            p = _frac_dec(a_codes[k]) * _frac_dec(b_codes[k])
            q = abs(p) // lsb * lsb
            total += q if p >= 0 else -q
    return total


def test_alignment_term_closed_forms():
    """Hand-worked runs: T = sum of min(|p|, grid) over the run's products off
    its grid 2^(E - 13), E the run's largest exponent sum."""
    A = np.zeros((1, 8), np.uint8)
    A[0, :2] = [0x60, 0x18]                       # 32 (exponent 5), 2^-4 (exponent -4)
    # products 1024 (E = 10, on the grid 2^-3) and 2^-8 (off it): T = 2^-8, the
    # device's actual loss for this run (1024 + 2^-8 -> 1024)
    assert gemm.alignment_term(A, A)[0, 0] == 2.0 ** -8
    Z = np.zeros((1, 16), np.uint8)               # all-zero runs lose nothing
    assert gemm.alignment_term(Z, Z)[0, 0] == 0.0
    sa, sb = np.array([2.0], np.float32), np.array([0.5], np.float32)
    assert gemm.alignment_term(A, A, sa, sb)[0, 0] == 2.0 ** -8
    sa3 = np.array([-3.0], np.float32)            # scales enter by magnitude
    assert gemm.alignment_term(A, A, sa3, sb)[0, 0] == 1.5 * 2.0 ** -8
    # 32*32 + 1.5*2^-3: the small product (3 * 2^-4) is off the grid 2^-3 and
    # larger than it, so it counts the grid: T = 2^-3 (the device loses 2^-4)
    a2 = np.array([[0x60, 0x3C] + [0] * 6], np.uint8)
    b2 = np.array([[0x60, 0x20] + [0] * 6], np.uint8)
    assert gemm.alignment_term(a2, b2)[0, 0] == 2.0 ** -3
    # 1.875^2 + 2^-6 * 2^-7: E = 0, grid 2^-13, and 2^-13 is on it: T = 0 (exact on the device)
    a3 = np.array([[0x3F, 0x08] + [0] * 6], np.uint8)
    b3 = np.array([[0x3F, 0x04] + [0] * 6], np.uint8)
    assert gemm.alignment_term(a3, b3)[0, 0] == 0.0
    # the same small product in the next run is on its own grid: T = 0
    a4 = np.zeros((1, 16), np.uint8)
    a4[0, 0], a4[0, 8] = 0x60, 0x18
    assert gemm.alignment_term(a4, a4)[0, 0] == 0.0
    # a ragged K: the last run is padded with zero codes
    a5 = np.array([[0x60, 0x18]], np.uint8)
    assert gemm.alignment_term(a5, a5)[0, 0] == 2.0 ** -8
    # mode (b): a run's loss times its block's factors 2^(130-127) 2^(130-127)
    A32 = np.zeros((1, 32), np.uint8)
    A32[0, :2] = [0x60, 0x18]
    e = np.array([[130]], np.uint8)
    assert gemm.alignment_term(A32, A32, ea=e, eb=e)[0, 0] == 2.0 ** -8 * 2.0 ** 6
    # E5M2: 0x50 = 32, 0x2C = 2^-4, the same run as the first case
    a6 = np.array([[0x50, 0x2C] + [0] * 6], np.uint8)
    assert gemm.alignment_term(a6, a6, fmt_a="e5m2", fmt_b="e5m2")[0, 0] == 2.0 ** -8


def test_alignment_term_is_per_output_element():
    """The term of one output depends on its own row and column only: it
    equals the term of that 1x1 problem."""
    A = synth.u8_codes(41, 1, (3, 40))
    B = synth.u8_codes(42, 2, (4, 40))
    T = gemm.alignment_term(A, B)
    for m in range(3):
        for n in range(4):
            assert T[m, n] == gemm.alignment_term(A[m:m + 1], B[n:n + 1])[0, 0]
    assert (T > 0).all()


def test_alignment_term_bounds_the_model():
    """The model's error never exceeds T, on random codes and on runs that mix
    magnitudes 2^13 apart; and the model reproduces the measured cases."""
    for seed in range(6):
        K = 8 * (3 + seed)
        A = synth.u8_codes(500 + seed, 1, (3, K))
        B = synth.u8_codes(600 + seed, 2, (2, K))
        T = gemm.alignment_term(A, B)
        for m in range(3):
            for n in range(2):
                exact = sum(_frac_dec(A[m, k]) * _frac_dec(B[n, k]) for k in range(K))
                err = abs(_emulate_group_alignment(A[m], B[n]) - exact)
                assert err <= Fraction(T[m, n]), (seed, m, n)
    # measured on the device: 1024 + 2^-8 in one run -> 1024; 2^10 + 3*2^-4 -> 1024.125
    a = np.array([0x60, 0x18] + [0] * 6, np.uint8)
    assert _emulate_group_alignment(a, a) == 1024
    a2 = np.array([0x60, 0x3C] + [0] * 6, np.uint8)   # 32, 1.5
    b2 = np.array([0x60, 0x20] + [0] * 6, np.uint8)   # 32, 2^-3: 1024 + 3*2^-4
    assert _emulate_group_alignment(a2, b2) == Fraction(1024125, 1000)
    a3 = np.array([0x60] + [0] * 7 + [0x18] + [0] * 7, np.uint8)   # the small product in the next run
    assert _emulate_group_alignment(a3, a3) == 1024 + Fraction(1, 256)


# ---- E5M2 operands (oracle.e5m2): the float64 sum rounds, within K * 2^-53 * W

from oracle import e5m2  # noqa: E402

FMT_PAIRS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


def _finite_codes(seed, shape, fmt):
    c = synth.u8_codes(seed, 1, shape, exclude_nan=False)
    if fmt == "e5m2":
        return np.where((c & 0x7C) == 0x7C, c & 0xF3, c).astype(np.uint8)   # drop Inf/NaN exponents
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


def _frac(c, fmt):
    return Fraction((e5m2 if fmt == "e5m2" else e4m3).decode_code(int(c)))


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 2, 48)])
def test_mode_a_rational_brute_force_e5m2(fa, fb, M, N, K):
    A = _finite_codes(700 + K, (M, K), fa)
    B = _finite_codes(800 + K, (N, K), fb)
    assert (e5m2.decode(A if fa == "e5m2" else B) != 0).any()
    sa = synth.scales(synth.WORKLOADS["c1_128x256x512"], "a")[:M]
    sb = synth.scales(synth.WORKLOADS["c1_128x256x512"], "b")[:N]
    D = gemm.gemm_scaled(A, B, sa, sb, fa, fb)
    W = gemm.gemm_scaled_weight(A, B, sa, sb, fa, fb)
    for m in range(M):
        for n in range(N):
            terms = [_frac(A[m, k], fa) * _frac(B[n, k], fb) for k in range(K)]
            s = Fraction(float(sa[m])) * Fraction(float(sb[n]))
            exact = sum(terms) * s
            absw = sum(abs(t) for t in terms) * abs(s)
            assert abs(Fraction(D[m, n]) - exact) <= (K + 2) * Fraction(1, 2 ** 53) * absw
            assert abs(Fraction(W[m, n]) - absw) <= (K + 2) * Fraction(1, 2 ** 53) * absw


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
def test_mode_b_rational_brute_force_e5m2(fa, fb):
    M, N, K = 2, 3, 96
    A = _finite_codes(900, (M, K), fa)
    B = _finite_codes(901, (N, K), fb)
    ea = synth.u8_codes(7, 2, (M, K // 32)) % 40 + 107
    eb = synth.u8_codes(8, 3, (N, K // 32)) % 40 + 107
    D = gemm.mxfp8_gemm(A, B, ea, eb, fa, fb)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(2) ** (int(ea[m, k // 32]) + int(eb[n, k // 32]) - 254)
                     * _frac(A[m, k], fa) * _frac(B[n, k], fb) for k in range(K)]
            absw = sum(abs(t) for t in terms)
            assert abs(Fraction(D[m, n]) - sum(terms)) <= (K + 2) * Fraction(1, 2 ** 53) * absw


def test_e5m2_product_table_every_code_pair():
    """Every pair of finite E5M2 codes, and every E4M3 x E5M2 pair, as a K=1
    product against torch's decode of both formats (products of 3-bit
    significands are exact in float64)."""
    c = np.arange(256, dtype=np.uint8)
    f5 = c[e5m2.is_finite_code(c)]
    f4 = c[e4m3.is_finite_code(c)]
    t5 = torch.from_numpy(f5).view(torch.float8_e5m2).to(torch.float64).numpy()
    t4 = torch.from_numpy(f4).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    one5, one4 = np.ones(f5.size, np.float32), np.ones(f4.size, np.float32)
    D = gemm.gemm_scaled(f5[:, None], f5[:, None], one5, one5, "e5m2", "e5m2")
    assert np.array_equal(D, np.outer(t5, t5))
    D = gemm.gemm_scaled(f4[:, None], f5[:, None], one4, one5, "e4m3", "e5m2")
    assert np.array_equal(D, np.outer(t4, t5))
    with pytest.raises(ValueError):
        gemm.gemm_scaled(np.array([[0x7C]], np.uint8), np.array([[0x3C]], np.uint8), one5[:1], one5[:1],
                         "e5m2", "e5m2")


def test_e5m2_ones_closed_form():
    """1.0 is 0x3C in E5M2: an all-ones product is K * sa * sb, also with an
    E4M3 1.0 (0x38) on the other side."""
    K = 1000
    A = np.full((2, K), 0x3C, np.uint8)
    B4 = np.full((3, K), 0x38, np.uint8)
    sa, sb = np.array([0.5, 3.0], np.float32), np.array([1.0, 2.0, 0.25], np.float32)
    assert np.array_equal(gemm.gemm_scaled(A, B4, sa, sb, "e5m2", "e4m3"), K * np.outer(sa, sb).astype(np.float64))


def test_alignment_term_e5m2_exponents():
    # 1.0 -> 0, max 57344 -> 15, min normal and every subnormal or zero -> -14
    c = np.array([0x3C, 0x7B, 0x04, 0x01, 0x00, 0x80, 0xBF], np.uint8)
    assert list(gemm.code_exponent(c, "e5m2")) == [0, 15, -14, -14, -14, -14, 0]
    Z = np.zeros((1, 16), np.uint8)                # all-zero runs lose nothing
    assert gemm.alignment_term(Z, Z, fmt_a="e5m2", fmt_b="e5m2")[0, 0] == 0.0
    A = np.zeros((1, 8), np.uint8)
    A[0, :2] = [0x50, 0x2C]                        # 32 = 2^5 and 2^-4 in E5M2
    B = np.zeros((1, 8), np.uint8)
    B[0, :2] = [0x60, 0x18]                        # 32 = 2^5 and 2^-4 in E4M3
    # products 1024 (E = 10) and 2^-8, which is off the grid 2^-3: T = 2^-8
    assert gemm.alignment_term(A, B, fmt_a="e5m2", fmt_b="e4m3")[0, 0] == 2.0 ** -8
    # 1 * 1 + 2^-16 * 2^-16 (E5M2 subnormals, exponent -14 each): E = 0, grid
    # 2^-13, the product 2^-32 is off it: T = 2^-32
    C = np.zeros((1, 8), np.uint8)
    C[0, :2] = [0x3C, 0x01]
    assert gemm.alignment_term(C, C, fmt_a="e5m2", fmt_b="e5m2")[0, 0] == 2.0 ** -32
