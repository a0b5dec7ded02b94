"""GPU parity of fp8_gemm_scaled (mode a) and mxfp8_gemm (mode b) vs the oracle.

Small and ragged shapes are compared on every element; the large workloads
(8192x2048x8192, the 8192x22016x8192 FFN-up projection, 4096x14336x4096 MXFP8)
run in the same launch configuration as the benchmark and are compared on
sampled rows x columns, each computed by the oracle from its own quantization
of those rows (the row-wise and MX quantizers are row-local).
Bound: |D - D_ref| <= 1e-5 * W + 1 ulp of the output format + T, where T is
the matrix-core alignment term (oracle.gemm: products in a run of 8 K values
are aligned to the run's largest exponent sum, 13 bits kept); each check also
reports how many elements meet the plain bound without T.
"""

import numpy as np
import pytest

import synth
from gpu_util import (assert_gemm_close, oracle_cast, oracle_mx_rows, oracle_quantize_rows, say, to_dev,
                      to_host)
from oracle import e4m3, gemm, quant

pytestmark = pytest.mark.gpu


def torch_dtype(out):
    import torch
    return torch.bfloat16 if out == "bf16" else torch.float32


def gpu_scaled(fp8g, A, B, sa, sb, out):
    M, K = A.shape
    N = B.shape[0]
    D = fp8g.fp8_gemm_scaled(M, N, K, to_dev(A), to_dev(B), to_dev(sa), to_dev(sb), out_dtype=torch_dtype(out))
    return to_host(D)


def gpu_mx(fp8g, A, B, ea, eb, out):
    M, K = A.shape
    N = B.shape[0]
    D = fp8g.mxfp8_gemm(M, N, K, to_dev(A), to_dev(B), to_dev(ea), to_dev(eb), out_dtype=torch_dtype(out))
    return to_host(D)


def codes(seed, shape, stream=1):
    return synth.u8_codes(seed, stream, shape)


def uscale(seed, n, stream=3):
    return (0.5 + 1.5 * synth.uniform(synth.stream_key(seed, stream), 0, n)).astype(np.float32)


# (M, N, K): tile-aligned, ragged in m/n, a K tail that is not a multiple of the
# 128-byte stage, single elements, several tiles in both directions.  Problems
# with at most half as many 256x256 tiles as CUs run on 128x128 tiles; 2561 x
# 3000 (11 x 12 tiles of 256) and larger take the 256x256 kernels, with ragged
# m, n and a K tail.  The epilogue depends on N: bf16 is staged through LDS for
# N % 8 == 0, fp32 for N % 32 == 0 (1000 x 1024, 2600 x 3072, 2561 x 3008);
# other N store from registers.  4864 x 4096 and 4864 x 4032 have 304 tiles
# of 256 for 256 workgroups: a workgroup runs a second tile, so its epilogue
# borrows a ring slot while the next tile's loads are in flight.  4352 x 4096
# (272 tiles of 256, just past one round) runs on 1088 tiles of 128.
SHAPES_A = [(1, 1, 16), (33, 65, 48), (256, 256, 128), (300, 200, 512), (257, 1000, 4112), (512, 768, 1024),
            (1, 513, 2048), (640, 3, 160), (1000, 1001, 272), (1000, 1024, 272), (2561, 3000, 272),
            (2561, 3008, 272), (2600, 2900, 1024), (2600, 3072, 1024), (4864, 4096, 256), (4864, 4032, 272),
            (4352, 4096, 272)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", SHAPES_A)
def test_mode_a_shapes(gpu_lib, M, N, K, out):
    seed = M * 7919 + N * 31 + K
    A, B = codes(seed, (M, K)), codes(seed, (N, K), 2)
    sa, sb = uscale(seed, M), uscale(seed, N, 4)
    say("mode a", M, N, K, out)
    D = gpu_scaled(gpu_lib, A, B, sa, sb, out)
    assert_gemm_close(D, gemm.gemm_scaled(A, B, sa, sb), gemm.gemm_scaled_weight(A, B, sa, sb), out,
                      "mode a %dx%dx%d %s" % (M, N, K, out), gemm.alignment_term(A, B, sa, sb))


@pytest.mark.parametrize("name", ["c1_128x256x512", "c2_2048x1024x4096"])
def test_mode_a_raw_cast_workloads(gpu_lib, name):
    """fp32 N(0,1) operands cast to E4M3 without scaling, U[0.5, 2] scales (the
    DeepGEMM call example and its benchmark shapes); every element compared."""
    w = synth.WORKLOADS[name]
    A, B = oracle_cast(synth.draw(w, "a")), oracle_cast(synth.draw(w, "b"))
    sa, sb = synth.scales(w, "a"), synth.scales(w, "b")
    say("mode a", name)
    D = gpu_scaled(gpu_lib, A, B, sa, sb, "bf16")
    assert D.shape == (w.M, w.N)
    _, plain_bad = assert_gemm_close(D, gemm.gemm_scaled(A, B, sa, sb), gemm.gemm_scaled_weight(A, B, sa, sb),
                                     "bf16", name, gemm.alignment_term(A, B, sa, sb))
    assert plain_bad == 0      # N(0,1) operands: the plain fp32-accumulation bound holds everywhere


# k = 0: every output is the empty sum.  The shapes take each epilogue path:
# from registers (N = 90), staged through LDS on 128-row tiles (300 x 512) and
# on 256-row tiles (2600 x 3072), for both output types.
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N", [(70, 90), (300, 512), (2600, 3072)])
def test_mode_a_k_zero(gpu_lib, M, N, out):
    import torch
    A = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    B = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    sa, sb = to_dev(uscale(1, M)), to_dev(uscale(2, N))
    D = torch.full((M, N), 5.0, dtype=torch_dtype(out), device="cuda")
    say("mode a k=0", M, N, out)
    gpu_lib.fp8_gemm_scaled(M, N, 0, A, B, sa, sb, D=D, out_dtype=torch_dtype(out))
    torch.cuda.synchronize()
    assert bool((D == 0).all())


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N", [(70, 90), (2600, 3072)])
def test_mode_b_k_zero(gpu_lib, M, N, out):
    import torch
    A = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    B = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    ea = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    eb = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    D = torch.full((M, N), 5.0, dtype=torch_dtype(out), device="cuda")
    say("mode b k=0", M, N, out)
    gpu_lib.mxfp8_gemm(M, N, 0, A, B, ea, eb, D=D, out_dtype=torch_dtype(out))
    torch.cuda.synchronize()
    assert bool((D == 0).all())


def test_mode_a_product_table(gpu_lib):
    """Every pair of finite codes: D = dec(a) dec(b) exactly (at most 8
    significant bits, so exact in bf16); pins the hardware decode of all codes."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for K, col in ((64, 0), (64, 63), (256, 200)):
        A = np.zeros((finite.size, K), np.uint8)
        B = np.zeros((finite.size, K), np.uint8)
        A[:, col] = finite
        B[:, col] = finite
        ones_m = np.ones(finite.size, np.float32)
        say("product table K", K, "col", col)
        D = gpu_scaled(gpu_lib, A, B, ones_m, ones_m, "bf16")
        dec = e4m3.decode(finite)
        assert np.array_equal(D, np.outer(dec, dec))


def test_mode_a_ones_closed_form(gpu_lib):
    M, N, K = 96, 80, 8192
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    say("ones closed form")
    D = gpu_scaled(gpu_lib, A, B, np.ones(M, np.float32), np.ones(N, np.float32), "f32")
    assert np.all(D == 8192.0)


def test_mode_a_one_hot_columns(gpu_lib):
    M, N, K = 130, 260, 384
    A = codes(77, (M, K))
    perm = (np.arange(N) * 37 + 5) % K
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), perm] = 0x38
    sa, sb = uscale(5, M), np.ones(N, np.float32)
    say("one-hot B")
    D = gpu_scaled(gpu_lib, A, B, sa, sb, "f32")
    want = e4m3.decode(A)[:, perm] * sa.astype(np.float64)[:, None]
    assert np.array_equal(D, want.astype(np.float32).astype(np.float64))


def _pipeline(fp8g, w, sample_m, sample_n):
    """GPU quantize -> GPU GEMM at full size, bf16 output (the benchmark's
    launch) and fp32 output (the staged fp32 epilogue); oracle on the sampled
    rows/cols."""
    import torch
    say("pipeline", w.name, "draw")
    XA, XB = synth.draw(w, "a"), synth.draw(w, "b")
    say("pipeline", w.name, "gpu")
    qa, sa = fp8g.fp8_quantize_rowwise(to_dev(XA))
    qb, sb = fp8g.fp8_quantize_rowwise(to_dev(XB))
    D = fp8g.fp8_gemm_scaled(w.M, w.N, w.K, qa, qb, sa, sb)
    torch.cuda.synchronize()
    Ds = {"bf16": to_host(D)[np.ix_(sample_m, sample_n)]}
    del D
    say("pipeline", w.name, "gpu f32")
    D = fp8g.fp8_gemm_scaled(w.M, w.N, w.K, qa, qb, sa, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Ds["f32"] = to_host(D)[np.ix_(sample_m, sample_n)]
    del D
    oa, osa = oracle_quantize_rows(XA[sample_m])
    ob, osb = oracle_quantize_rows(XB[sample_n])
    # the GPU codes on the sampled rows must be the oracle's, bit for bit
    assert np.array_equal(to_host(qa)[sample_m], oa) and np.array_equal(to_host(sa)[sample_m], osa)
    assert np.array_equal(to_host(qb)[sample_n], ob) and np.array_equal(to_host(sb)[sample_n], osb)
    ref = gemm.gemm_scaled(oa, ob, osa, osb)
    W = gemm.gemm_scaled_weight(oa, ob, osa, osb)
    T = gemm.alignment_term(oa, ob, osa, osb)
    for out in ("bf16", "f32"):
        assert_gemm_close(Ds[out], ref, W, out, "%s %s" % (w.name, out), T)


def _samples(total, n, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(total, size=n - 4, replace=False).tolist()) | {0, 255, 256, total - 1}
    return np.array(sorted(idx))


def test_mode_a_c3_pipeline(gpu_lib):
    w = synth.WORKLOADS["c3_8192x2048x8192"]
    _pipeline(gpu_lib, w, _samples(w.M, 96, 1), _samples(w.N, 256, 2))


def test_mode_a_ffn_up_pipeline(gpu_lib):
    w = synth.WORKLOADS["c4_ffn_up_8192x22016x8192"]
    _pipeline(gpu_lib, w, _samples(w.M, 64, 3), _samples(w.N, 512, 4))


def test_mode_a_deterministic(gpu_lib):
    import torch
    M, N, K = 1024, 1280, 2048
    A, B = to_dev(codes(9, (M, K))), to_dev(codes(9, (N, K), 2))
    sa, sb = to_dev(uscale(9, M)), to_dev(uscale(9, N))
    D1 = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
    D2 = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


# ------------------------------------------------------------------ mode (b)

def mx_scales(seed, R, nb, stream):
    return (synth.u8_codes(seed, stream, (R, nb), exclude_nan=False) % 41 + 107).astype(np.uint8)


SHAPES_B = [(32, 32, 32), (64, 96, 96), (256, 256, 256), (257, 300, 4128), (512, 512, 1024), (5, 700, 160),
            (300, 7, 64), (2561, 3000, 1056), (2600, 2900, 1024)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", SHAPES_B)
def test_mode_b_shapes(gpu_lib, M, N, K, out):
    seed = M * 131 + N * 17 + K
    A, B = codes(seed, (M, K)), codes(seed, (N, K), 2)
    ea, eb = mx_scales(seed, M, K // 32, 7), mx_scales(seed, N, K // 32, 8)
    say("mode b", M, N, K, out)
    D = gpu_mx(gpu_lib, A, B, ea, eb, out)
    assert_gemm_close(D, gemm.mxfp8_gemm(A, B, ea, eb), gemm.mxfp8_gemm_weight(A, B, ea, eb), out,
                      "mode b %dx%dx%d %s" % (M, N, K, out), gemm.alignment_term(A, B, ea=ea, eb=eb))


def test_mode_b_scale_association(gpu_lib):
    """Only block j carries data (one product per output): D = 2^(ea+eb-254) dec dec
    exactly.  Pins which scale byte the hardware applies to which 32-element block,
    for every block position inside a 128-byte stage and for both lane halves."""
    M, N, K = 64, 64, 256
    base_a = np.array([0x38, 0x7E, 0x81, 0xB9] * 16, np.uint8)
    base_b = np.array([0x40, 0xB9, 0x01, 0x7E] * 16, np.uint8)
    for j in range(K // 32):
        for t in (0, 17, 31):
            A = np.zeros((M, K), np.uint8)
            B = np.zeros((N, K), np.uint8)
            A[:, 32 * j + t] = base_a
            B[:, 32 * j + t] = base_b
            ea = np.full((M, K // 32), 127, np.uint8)
            eb = np.full((N, K // 32), 127, np.uint8)
            ea[:, j] = 100 + (np.arange(M) % 50)
            eb[:, j] = 110 + (np.arange(N) * 3 % 40)
            # poison the other blocks' scales so a wrong association shows up
            for jj in range(K // 32):
                if jj != j:
                    ea[:, jj] = 140
                    eb[:, jj] = 90
            say("mx association block", j, "t", t)
            D = gpu_mx(gpu_lib, A, B, ea, eb, "f32")
            want = np.outer(e4m3.decode(base_a) * quant.ue8m0_value(ea[:, j]),
                            e4m3.decode(base_b) * quant.ue8m0_value(eb[:, j]))
            assert np.array_equal(D, want), (j, t)


# Neutral block scales (code 127) make mode (b) compute mode (a) with unit
# scales through the same matrix-core instruction, so the two must agree bit
# for bit.  On 4864 x 4096 (304 tiles of 256, two per workgroup for some) the
# fp32 outputs come from different epilogues -- staged through LDS in mode (a),
# from registers in mode (b) -- which this compares exactly.
@pytest.mark.parametrize("M,N,K,out", [(300, 260, 1024, "f32"), (4864, 4096, 1024, "f32"),
                                       (4864, 4096, 1024, "bf16")])
def test_mode_b_neutral_scales_equal_mode_a(gpu_lib, M, N, K, out):
    A, B = codes(3, (M, K)), codes(3, (N, K), 2)
    ea = np.full((M, K // 32), 127, np.uint8)
    eb = np.full((N, K // 32), 127, np.uint8)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    say("mx neutral vs mode a", M, N, K, out)
    Dx = gpu_mx(gpu_lib, A, B, ea, eb, out)
    Da = gpu_scaled(gpu_lib, A, B, ones_m, ones_n, out)
    assert np.array_equal(Dx, Da)
    sm = np.union1d(np.arange(0, M, 37), [M - 1])
    assert_gemm_close(Dx[sm], gemm.gemm_scaled(A[sm], B, ones_m[sm], ones_n),
                      gemm.gemm_scaled_weight(A[sm], B, ones_m[sm], ones_n), out, "mx neutral",
                      gemm.alignment_term(A[sm], B))


def test_mode_b_mx_workload(gpu_lib):
    """4096x14336x4096 MXFP8: N(0,1) x 2^u per 32-block, quantized with the MX
    rule (oracle, host) -> GPU GEMM at full size; sampled rows x cols checked."""
    import torch
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    say("mx workload draw")
    qa, ea = oracle_mx_rows(synth.draw(w, "a"))
    qb, eb = oracle_mx_rows(synth.draw(w, "b"))
    sm, sn = _samples(w.M, 64, 5), _samples(w.N, 384, 6)
    ref = gemm.mxfp8_gemm(qa[sm], qb[sn], ea[sm], eb[sn])
    W = gemm.mxfp8_gemm_weight(qa[sm], qb[sn], ea[sm], eb[sn])
    T = gemm.alignment_term(qa[sm], qb[sn], ea=ea[sm], eb=eb[sn])
    A, B, EA, EB = to_dev(qa), to_dev(qb), to_dev(ea), to_dev(eb)
    for out in ("bf16", "f32"):   # the benchmark's launch, and fp32 output from registers
        say("mx workload gpu", out)
        D = gpu_lib.mxfp8_gemm(w.M, w.N, w.K, A, B, EA, EB, out_dtype=torch_dtype(out))
        torch.cuda.synchronize()
        assert_gemm_close(to_host(D)[np.ix_(sm, sn)], ref, W, out, "%s %s" % (w.name, out), T)
        del D


# Whole scale dwords (K % 128 == 0): the scales of 4 stages at a time are
# staged together, so the last group of a tile is partial unless the stages
# per tile (K / 128) are a multiple of 4, and with more tiles than workgroups
# a workgroup's next tile's first group is loaded during its current tile.
# 4352 x 4096: 272 tiles of 256 for 256 workgroups; 2048 x 4096: 128 tiles of
# 256, so 512 tiles of 128 (two per workgroup).  Rows and columns sampled at
# a stride cover every tile.
SHAPES_B_GROUPS = [(4352, 4096, 128), (4352, 4096, 384), (4352, 4096, 640), (4352, 4096, 1664),
                   (2048, 4096, 640), (2048, 4096, 896)]


@pytest.mark.parametrize("M,N,K", SHAPES_B_GROUPS)
def test_mode_b_scale_groups(gpu_lib, M, N, K):
    seed = M + 7 * N + 3 * K
    A, B = codes(seed, (M, K)), codes(seed, (N, K), 2)
    ea, eb = mx_scales(seed, M, K // 32, 7), mx_scales(seed, N, K // 32, 8)
    say("mode b scale groups", M, N, K)
    D = gpu_mx(gpu_lib, A, B, ea, eb, "bf16")
    sm = np.union1d(np.arange(0, M, 13), [M - 1])
    sn = np.union1d(np.arange(0, N, 11), [N - 1])
    assert_gemm_close(D[np.ix_(sm, sn)], gemm.mxfp8_gemm(A[sm], B[sn], ea[sm], eb[sn]),
                      gemm.mxfp8_gemm_weight(A[sm], B[sn], ea[sm], eb[sn]), "bf16",
                      "mode b groups %dx%dx%d" % (M, N, K), gemm.alignment_term(A[sm], B[sn], ea=ea[sm], eb=eb[sn]))
