"""Pins for the plain C++ oracle (oracle/cpp/fp8_oracle.cpp), CPU only.

  * The cast on every one of the 2^32 fp32 bit patterns, E4M3 and E5M2: the
    definition (nearest decoded magnitude, ties to the even code, saturating)
    against an independent integer bit-manipulation of the same rounding.
  * The two oracles (C++ and numpy) against each other: the 256-entry decode
    tables, the cast on random patterns and on every rounding boundary, the
    row-wise quantizer (bit for bit) and both GEMM modes.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import cpp_oracle, e4m3, e5m2, gemm, quant

FMTS = {"e4m3": e4m3, "e5m2": e5m2}


def test_decode_tables_agree():
    for name, mod in FMTS.items():
        t = cpp_oracle.decode_table(name)
        ref = mod.DECODE_TABLE
        assert np.array_equal(np.isnan(t), np.isnan(ref)), name
        ok = ~np.isnan(ref)
        assert np.array_equal(t[ok], ref[ok]), name
        assert np.array_equal(np.signbit(t[ok]), np.signbit(ref[ok])), name


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_cast_every_fp32_pattern(fmt):
    """All 2^32 patterns: the definitional cast equals the bit-level cast."""
    chunk = 1 << 26
    starts = range(0, 1 << 32, chunk)
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as pool:
        res = list(pool.map(lambda lo: (lo, cpp_oracle.cast_sweep(lo, lo + chunk, fmt)), starts))
    bad = [(lo, r) for lo, r in res if r[0]]
    assert not bad, "first mismatching pattern 0x%08x (%d in that chunk)" % (bad[0][1][1], bad[0][1][0])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_cast_agrees_with_numpy_oracle(fmt):
    mod = FMTS[fmt]
    rng = np.random.default_rng(5)
    x = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = x[~np.isnan(x)]
    mags = mod.DECODE_TABLE[:mod.MAX_CODE + 1]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    x = np.concatenate([x, near, -near, np.float32([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45])])
    assert np.array_equal(cpp_oracle.encode(x, fmt), mod.encode(x))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_rowwise_agrees(fmt):
    w = synth.WORKLOADS["c4_ffn_up_8192x22016x8192"]
    x = synth.draw(w, "a", slice(0, 48))[:, :1000].copy()
    t = np.float32(2.0 ** -149)
    x[0] = 0.0
    x[1, :3] = [t, -t, 0.0]
    x[2] *= np.float32(1e-36)
    x[3] *= np.float32(1e30)
    q1, s1 = cpp_oracle.quantize_rowwise(x, fmt)
    q2, s2 = quant.quantize_rowwise(x, fmt)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q1, q2)


def _codes(seed, shape, fmt):
    c = synth.u8_codes(seed, 1, shape, exclude_nan=False)
    if fmt == "e5m2":
        return np.where((c & 0x7C) == 0x7C, c & 0xF3, c).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_gemms_agree(fa, fb):
    M, N, K = 7, 9, 160
    A, B = _codes(31, (M, K), fa), _codes(32, (N, K), fb)
    sa = (0.5 + synth.uniform(synth.stream_key(33, 1), 0, M)).astype(np.float32)
    sb = (0.5 + synth.uniform(synth.stream_key(33, 2), 0, N)).astype(np.float32)
    D1 = cpp_oracle.gemm_scaled(A, B, sa, sb, fa, fb)
    D2 = gemm.gemm_scaled(A, B, sa, sb, fa, fb)
    W = gemm.gemm_scaled_weight(A, B, sa, sb, fa, fb)
    if fa == fb == "e4m3":
        assert np.array_equal(D1, D2)          # both exact sums, the same two roundings
    else:
        assert np.all(np.abs(D1 - D2) <= (2 * K + 4) * 2.0 ** -53 * W)
    ea = (synth.u8_codes(34, 3, (M, K // 32)) % 41 + 107).astype(np.uint8)
    eb = (synth.u8_codes(35, 4, (N, K // 32)) % 41 + 107).astype(np.uint8)
    X1 = cpp_oracle.mxfp8_gemm(A, B, ea, eb, fa, fb)
    X2 = gemm.mxfp8_gemm(A, B, ea, eb, fa, fb)
    XW = gemm.mxfp8_gemm_weight(A, B, ea, eb, fa, fb)
    assert np.all(np.abs(X1 - X2) <= (2 * K + 4) * 2.0 ** -53 * XW)


@pytest.mark.parametrize("fmt_a,fmt_b", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_cpp_alignment_term_matches_numpy(fmt_a, fmt_b):
    """The threaded C++ loop computes the numpy oracle's matrix-core term (mode
    (a) with scales, mode (b) with block factors, a ragged K)."""
    def finite(seed, shape, fmt):
        c = synth.u8_codes(seed, 1, shape, exclude_nan=False)
        if fmt == "e5m2":
            return np.where((c & 0x7C) == 0x7C, c & 0xF3, c).astype(np.uint8)
        return np.where((c & 0x7F) == 0x7F, c & 0xF7, c).astype(np.uint8)
    A, B = finite(11, (5, 72), fmt_a), finite(12, (7, 72), fmt_b)
    sa = (0.5 + synth.uniform(synth.stream_key(13, 3), 0, 5)).astype(np.float32)
    sb = (0.5 + synth.uniform(synth.stream_key(13, 4), 0, 7)).astype(np.float32)
    for args in ((), (sa, sb)):
        ref = gemm.alignment_term(A, B, *args, fmt_a=fmt_a, fmt_b=fmt_b)
        got = cpp_oracle.alignment_term(A, B, *args, fmt_a=fmt_a, fmt_b=fmt_b, threads=3)
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)
    A, B = A[:, :64], B[:, :64]
    ea = (synth.u8_codes(14, 7, (5, 2), exclude_nan=False) % 21 + 117).astype(np.uint8)
    eb = (synth.u8_codes(14, 8, (7, 2), exclude_nan=False) % 21 + 117).astype(np.uint8)
    ref = gemm.alignment_term(A, B, ea=ea, eb=eb, fmt_a=fmt_a, fmt_b=fmt_b)
    got = cpp_oracle.alignment_term(A, B, ea=ea, eb=eb, fmt_a=fmt_a, fmt_b=fmt_b)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)


def test_mx_quantize_agrees():
    """The C++ MX block quantizer against the numpy oracle's (two independent
    restatements of the MXFP8 page's rule), bit for bit, on the MX workload's
    recipe and on edge blocks; plus one block worked by hand: 32 ones have
    amax 1, the smallest e with 1 <= 448 * 2^e is -8 (448/256 = 1.75, 448/512
    = 0.875), so the scale code is 127 - 8 = 119 and every element is
    1 * 2^8 = 256 = 2^8, E4M3 exponent field 8 + 7 = 15, mantissa 0: 0x78."""
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    x = synth.draw(w, "a", slice(0, 24))[:, :1024].copy()
    x[0, :32] = 1.0                                   # the hand-worked block
    x[1, :32] = 0.0                                   # all zero: e = -127
    x[1, 32:64] = 448.0                               # amax exactly 448: e = 0
    x[1, 64:96] = np.float32(448.0 * 8)               # exactly 448 * 2^3: e = 3
    x[1, 96] = np.nextafter(np.float32(448.0), np.float32(1e9))   # just above 448: e = 1
    x[1, 128:160] = np.float32(2.0 ** -149)           # fp32 subnormal: e = -127, codes 0
    x[1, 160:192] *= np.float32(1e-30)
    x[1, 192:224] *= np.float32(1e30)
    q1, e1 = cpp_oracle.mx_quantize(x, threads=3)
    q2, e2 = quant.mx_quantize(x)
    assert np.array_equal(e1, e2) and np.array_equal(q1, q2)
    assert (q1[0, :32] == 0x78).all() and e1[0, 0] == 119
    assert e1[1, 0] == 0 and e1[1, 1] == 127 and e1[1, 2] == 130 and e1[1, 3] == 128 and e1[1, 4] == 0
    assert (q1[1, 128:160] == 0).all()


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_gemm_weight_and_threads(fa, fb):
    """The C++ GEMMs' bound weight W equals the numpy oracle's (exactly for
    E4M3 x E4M3, whose |product| sums are exact in double), and the results
    do not depend on the number of threads."""
    M, N, K = 6, 11, 224
    A, B = _codes(41, (M, K), fa), _codes(42, (N, K), fb)
    sa = (0.5 + synth.uniform(synth.stream_key(43, 1), 0, M)).astype(np.float32)
    sb = (0.5 + synth.uniform(synth.stream_key(43, 2), 0, N)).astype(np.float32)
    D1, W1 = cpp_oracle.gemm_scaled(A, B, sa, sb, fa, fb, weight=True, threads=1)
    D5, W5 = cpp_oracle.gemm_scaled(A, B, sa, sb, fa, fb, weight=True, threads=5)
    assert np.array_equal(D1, D5) and np.array_equal(W1, W5)
    Wn = gemm.gemm_scaled_weight(A, B, sa, sb, fa, fb)
    if fa == fb == "e4m3":
        assert np.array_equal(W1, Wn)
    np.testing.assert_allclose(W1, Wn, rtol=1e-13, atol=0)
    ea = (synth.u8_codes(44, 3, (M, K // 32)) % 41 + 107).astype(np.uint8)
    eb = (synth.u8_codes(45, 4, (N, K // 32)) % 41 + 107).astype(np.uint8)
    X1, XW1 = cpp_oracle.mxfp8_gemm(A, B, ea, eb, fa, fb, weight=True, threads=1)
    X4, XW4 = cpp_oracle.mxfp8_gemm(A, B, ea, eb, fa, fb, weight=True, threads=4)
    assert np.array_equal(X1, X4) and np.array_equal(XW1, XW4)
    np.testing.assert_allclose(XW1, gemm.mxfp8_gemm_weight(A, B, ea, eb, fa, fb), rtol=1e-13, atol=0)
    q1, s1 = cpp_oracle.quantize_rowwise(synth.draw(synth.WORKLOADS["c3_8192x2048x8192"], "a", slice(0, 9)), threads=1)
    q4, s4 = cpp_oracle.quantize_rowwise(synth.draw(synth.WORKLOADS["c3_8192x2048x8192"], "a", slice(0, 9)), threads=4)
    assert np.array_equal(q1, q4) and np.array_equal(s1.view(np.uint32), s4.view(np.uint32))
