"""GPU parity of the format-per-operand GEMMs (fp8_gemm_scaled_ex,
mxfp8_gemm_ex) with E5M2 operands vs the oracle (oracle.gemm with fmt_a /
fmt_b, decode from oracle.e5m2).

Bound as for E4M3: |D - D_ref| <= 1e-5 * W + 1 ulp of the output + T, with
the alignment term T taken from each operand's own exponent field (E5M2:
bias 15, subnormals at -14).  The matrix core treats E5M2 products like E4M3
ones -- runs of 8 aligned to the largest exponent sum, 13 bits kept (the
measured cases are in test_gpu_matrix_core.py).
"""

import numpy as np
import pytest

import synth
from gpu_util import alignment, assert_gemm_close, say, to_dev, to_host
from oracle import e4m3, e5m2, gemm, quant

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
NAME = {E4M3: "e4m3", E5M2: "e5m2"}
PAIRS = [(E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3)]


def torch_dtype(out):
    import torch
    return torch.bfloat16 if out == "bf16" else torch.float32


def finite_codes(seed, shape, fmt, stream=1):
    """Uniform random bytes with the non-finite codes of the format remapped
    (E5M2: exponent field 31 -> 28; E4M3: NaN -> its neighbour)."""
    c = synth.u8_codes(seed, stream, shape, exclude_nan=False)
    if fmt == E5M2:
        return np.where((c & 0x7C) == 0x7C, c & 0xF3, c).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


def uscale(seed, n, stream=3):
    return (0.5 + 1.5 * synth.uniform(synth.stream_key(seed, stream), 0, n)).astype(np.float32)


def gpu_scaled_ex(fp8g, A, fa, B, fb, sa, sb, out):
    M, K = A.shape
    N = B.shape[0]
    return to_host(fp8g.fp8_gemm_scaled_ex(M, N, K, to_dev(A), fa, to_dev(B), fb, to_dev(sa), to_dev(sb),
                                           out_dtype=torch_dtype(out)))


def gpu_mx_ex(fp8g, A, fa, B, fb, ea, eb, out):
    M, K = A.shape
    N = B.shape[0]
    return to_host(fp8g.mxfp8_gemm_ex(M, N, K, to_dev(A), fa, to_dev(B), fb, to_dev(ea), to_dev(eb),
                                      out_dtype=torch_dtype(out)))


def check_scaled(fp8g, A, fa, B, fb, sa, sb, out, what):
    say(what)
    D = gpu_scaled_ex(fp8g, A, fa, B, fb, sa, sb, out)
    na, nb = NAME[fa], NAME[fb]
    return assert_gemm_close(D, gemm.gemm_scaled(A, B, sa, sb, na, nb), gemm.gemm_scaled_weight(A, B, sa, sb, na, nb),
                             out, what, alignment(A, B, sa, sb, fmt_a=na, fmt_b=nb))


# on a 256-CU part the shapes up to 1000 x 1001 run on 64x128 tiles, 1900 x
# 2000 (240 tiles of 128) on 128x128 tiles, 2561 x 3000 (more than half as
# many 256x256 tiles as CUs) on 256x256 tiles and 2600 x 2904 (132 tiles of
# 256x256, 253 of 256x128) on 256x128 tiles
SHAPES_A = [(1, 1, 16), (33, 65, 48), (256, 256, 128), (300, 200, 512), (257, 1000, 4112), (1, 513, 2048),
            (1000, 1001, 272), (1900, 2000, 1024), (2561, 3000, 272), (2600, 2904, 1056)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES_A)
def test_ex_mode_a_random_codes(gpu_lib, M, N, K, fa, fb, out):
    """Uniform random codes: E5M2 products over 2^-32 .. 2^30 in every K run."""
    seed = M * 7919 + N * 31 + K + 101 * (2 * fa + fb)
    A, B = finite_codes(seed, (M, K), fa), finite_codes(seed, (N, K), fb, 2)
    check_scaled(gpu_lib, A, fa, B, fb, uscale(seed, M), uscale(seed, N, 4), out,
                 "ex mode a %s x %s %dx%dx%d %s" % (NAME[fa], NAME[fb], M, N, K, out))


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_ex_mode_a_raw_cast(gpu_lib, fa, fb):
    """The 2048x1024x4096 DeepGEMM call shape: N(0,1) values cast to each
    operand's format without scaling, U[0.5, 2] scales; every element."""
    w = synth.WORKLOADS["c2_2048x1024x4096"]
    enc = {E4M3: e4m3.encode, E5M2: e5m2.encode}
    A, B = enc[fa](synth.draw(w, "a")), enc[fb](synth.draw(w, "b"))
    _, plain_bad = check_scaled(gpu_lib, A, fa, B, fb, synth.scales(w, "a"), synth.scales(w, "b"), "bf16",
                                "ex raw cast %s x %s %s" % (NAME[fa], NAME[fb], w.name))
    assert plain_bad == 0      # N(0,1) operands: the plain fp32-accumulation bound holds everywhere


def test_ex_product_tables(gpu_lib):
    """Every pair of finite E5M2 codes, and every E4M3 x E5M2 pair, one product
    per output (3-bit x 3-bit significands: exact in bf16): pins the hardware's
    decode of every E5M2 code, in either operand position."""
    c = np.arange(256, dtype=np.uint8)
    f5, f4 = c[e5m2.is_finite_code(c)], c[e4m3.is_finite_code(c)]
    for (fa, ca), (fb, cb) in (((E5M2, f5), (E5M2, f5)), ((E4M3, f4), (E5M2, f5)), ((E5M2, f5), (E4M3, f4))):
        for K, col in ((64, 0), (64, 45), (256, 200)):
            A = np.zeros((ca.size, K), np.uint8)
            B = np.zeros((cb.size, K), np.uint8)
            A[:, col], B[:, col] = ca, cb
            say("ex product table", NAME[fa], NAME[fb], "K", K, "col", col)
            D = gpu_scaled_ex(gpu_lib, A, fa, B, fb, np.ones(ca.size, np.float32), np.ones(cb.size, np.float32),
                              "bf16")
            dec = {E4M3: e4m3.decode, E5M2: e5m2.decode}
            assert np.array_equal(D, np.outer(dec[fa](ca), dec[fb](cb))), (fa, fb, K, col)


def test_ex_e4m3_pair_is_the_plain_call(gpu_lib):
    """Both formats E4M3: the _ex calls give the plain calls' results bit for bit."""
    import torch
    M, N, K = 300, 520, 1024
    A = to_dev(finite_codes(5, (M, K), E4M3))
    B = to_dev(finite_codes(5, (N, K), E4M3, 2))
    sa, sb = to_dev(uscale(5, M)), to_dev(uscale(5, N))
    say("ex e4m3 pair vs plain")
    D1 = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
    D2 = gpu_lib.fp8_gemm_scaled_ex(M, N, K, A, E4M3, B, E4M3, sa, sb)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    ea = to_dev((synth.u8_codes(6, 7, (M, K // 32)) % 41 + 107).astype(np.uint8))
    eb = to_dev((synth.u8_codes(6, 8, (N, K // 32)) % 41 + 107).astype(np.uint8))
    D1 = gpu_lib.mxfp8_gemm(M, N, K, A, B, ea, eb)
    D2 = gpu_lib.mxfp8_gemm_ex(M, N, K, A, E4M3, B, E4M3, ea, eb)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


def test_ex_dtype_checks(gpu_lib):
    """float8 tensors must match the format they are declared as."""
    import torch
    A = torch.zeros((4, 64), dtype=torch.float8_e4m3fn, device="cuda")
    B = torch.zeros((4, 64), dtype=torch.float8_e5m2, device="cuda")
    s = torch.ones(4, device="cuda")
    D = gpu_lib.fp8_gemm_scaled_ex(4, 4, 64, A, E4M3, B, E5M2, s, s)
    assert bool((D == 0).all())
    with pytest.raises(TypeError):
        gpu_lib.fp8_gemm_scaled_ex(4, 4, 64, A, E5M2, B, E5M2, s, s)
    with pytest.raises(ValueError):
        gpu_lib.fp8_gemm_scaled_ex(4, 4, 64, A.view(torch.uint8), 2, B, E5M2, s, s)


# K / 128 = 3 and 5: the last group of 4 stages' block scales is partial.  On
# a 256-CU part 2600 x 2900 runs on 256x128 tiles (with and without a K tail)
# and 2304 x 4000 (K tail) on 256x256 tiles; the rest on 128x128 tiles.
SHAPES_B = [(32, 32, 32), (64, 96, 96), (257, 300, 4128), (512, 512, 1024), (5, 700, 160), (2600, 2900, 1024),
            (2600, 2900, 1056), (2304, 4000, 160), (300, 260, 384), (200, 300, 640)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES_B)
def test_ex_mode_b_random_codes(gpu_lib, M, N, K, fa, fb, out):
    seed = M * 131 + N * 17 + K + 7 * (2 * fa + fb)
    A, B = finite_codes(seed, (M, K), fa), finite_codes(seed, (N, K), fb, 2)
    ea = (synth.u8_codes(seed, 7, (M, K // 32)) % 41 + 107).astype(np.uint8)
    eb = (synth.u8_codes(seed, 8, (N, K // 32)) % 41 + 107).astype(np.uint8)
    what = "ex mode b %s x %s %dx%dx%d %s" % (NAME[fa], NAME[fb], M, N, K, out)
    say(what)
    D = gpu_mx_ex(gpu_lib, A, fa, B, fb, ea, eb, out)
    na, nb = NAME[fa], NAME[fb]
    assert_gemm_close(D, gemm.mxfp8_gemm(A, B, ea, eb, na, nb), gemm.mxfp8_gemm_weight(A, B, ea, eb, na, nb), out,
                      what, alignment(A, B, ea=ea, eb=eb, fmt_a=na, fmt_b=nb))


def test_ex_mode_b_scale_association_e5m2(gpu_lib):
    """One populated 32-block per call, E5M2 x E4M3: D = 2^(ea+eb-254) dec dec
    exactly, for every block of a 128-byte stage."""
    M, N, K = 64, 64, 256
    base_a = np.array([0x3C, 0x7B, 0x81, 0xBD] * 16, np.uint8)     # E5M2: 1, 57344, -2^-16, -1.25
    base_b = np.array([0x40, 0xB9, 0x01, 0x7E] * 16, np.uint8)     # E4M3
    for j in range(K // 32):
        A = np.zeros((M, K), np.uint8)
        B = np.zeros((N, K), np.uint8)
        A[:, 32 * j + 7] = base_a
        B[:, 32 * j + 7] = base_b
        ea = np.full((M, K // 32), 140, np.uint8)
        eb = np.full((N, K // 32), 90, np.uint8)
        ea[:, j] = 100 + (np.arange(M) % 50)
        eb[:, j] = 110 + (np.arange(N) * 3 % 40)
        say("ex mx association block", j)
        D = gpu_mx_ex(gpu_lib, A, E5M2, B, E4M3, ea, eb, "f32")
        want = np.outer(e5m2.decode(base_a) * quant.ue8m0_value(ea[:, j]),
                        e4m3.decode(base_b) * quant.ue8m0_value(eb[:, j]))
        assert np.array_equal(D, want), j


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 640), (4096, 8192, 640)])
def test_ex_mode_b_scale_groups_e5m2(gpu_lib, M, N, K):
    """E5M2 x E5M2 MX with 5 stages per tile (a partial last group of 4
    stages' block scales, and groups loaded for a workgroup's next tile), on
    544 tiles of 256x128 (4352 x 4096) and 512 of 256x256 (4096 x 8192) for
    256 workgroups; rows and columns sampled at a stride cover every tile."""
    seed = 99
    A, B = finite_codes(seed, (M, K), E5M2), finite_codes(seed, (N, K), E5M2, 2)
    ea = (synth.u8_codes(seed, 7, (M, K // 32)) % 41 + 107).astype(np.uint8)
    eb = (synth.u8_codes(seed, 8, (N, K // 32)) % 41 + 107).astype(np.uint8)
    say("ex mode b scale groups e5m2", M, N, K)
    D = gpu_mx_ex(gpu_lib, A, E5M2, B, E5M2, ea, eb, "bf16")
    sm = np.union1d(np.arange(0, M, 13), [M - 1])
    sn = np.union1d(np.arange(0, N, 11), [N - 1])
    a, b, sa_, sb_ = A[sm], B[sn], ea[sm], eb[sn]
    assert_gemm_close(D[np.ix_(sm, sn)], gemm.mxfp8_gemm(a, b, sa_, sb_, "e5m2", "e5m2"),
                      gemm.mxfp8_gemm_weight(a, b, sa_, sb_, "e5m2", "e5m2"), "bf16", "ex mode b groups e5m2",
                      alignment(a, b, ea=sa_, eb=sb_, fmt_a="e5m2", fmt_b="e5m2"))
