"""GPU results against the plain C++ oracle (oracle/cpp/fp8_oracle.cpp).

The C++ oracle decodes every FP8 code from the format's bit fields, casts by
the round-to-nearest-even definition (checked on every fp32 bit pattern by the
CPU tests) and sums in double.  Here it is the reference of the library's
results:
  * the row-wise quantizer (E4M3 and E5M2 output) and the MX block quantizer,
    bit for bit;
  * both GEMM modes within 1e-5 W + 1 ulp + T, W the C++ oracle's weight and
    T the matrix-core truncation term (the C++ loop of oracle.gemm's
    definition), at ragged shapes on every tile shape (64x128, 128x128, split
    over K, 256x128, 256x256) with every element compared;
  * the full-size workloads in the benchmark's launch configurations (also
    the FFN-up step with E5M2 operands): the GPU's quantized operands against
    the C++ quantizers' (activations on the sampled rows, weights on every
    row), and D on one row in every 128-row band against every column, with
    ceilings on the elements over the plain bound (test_gpu_gemm's for E4M3).
Every input comes from the seeded generators and the C++ quantizers, none from
the GPU.
"""

import numpy as np
import pytest

import synth
from gpu_util import alignment, assert_gemm_close, say, to_dev, to_host
from oracle import cpp_oracle
from test_gpu_gemm import PLAIN_MAX, band_rows

pytestmark = pytest.mark.gpu

# Elements over the plain bound (T = 0) on the sampled rows of the FFN-up step
# with E5M2 operands, recorded with margin: 5 (bf16) and 1077 (fp32) of 1453056.
PLAIN_MAX_E5M2 = {"bf16": 8, "f32": 1200}


def _codes(t):
    import torch
    return t.view(torch.uint8).cpu().numpy()


def _uscale(seed, n, stream):
    return (0.5 + 1.5 * synth.uniform(synth.stream_key(seed, stream), 0, n)).astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_rowwise_matches_cpp(gpu_lib, fmt):
    w = synth.WORKLOADS["c4_ffn_up_8192x22016x8192"]
    x = synth.draw(w, "a", slice(0, 768)).copy()
    t = np.float32(2.0 ** -149)
    x[0] = 0.0
    x[1, :3] = [t, -t, 0.0]
    x[2] *= np.float32(1e-36)
    x[3] *= np.float32(1e30)
    x[4, 7] = np.float32(-3.0e38)
    say("quantize vs C++", fmt)
    q, s = gpu_lib.fp8_quantize_ex(to_dev(x), fmt=gpu_lib.FMT_E5M2 if fmt == "e5m2" else gpu_lib.FMT_E4M3)
    cq, cs = cpp_oracle.quantize_rowwise(x, fmt)
    assert np.array_equal(to_host(s).view(np.uint32), cs.view(np.uint32))
    assert np.array_equal(_codes(q), cq)


def test_mx_quantize_matches_cpp(gpu_lib):
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    x = synth.draw(w, "b", slice(0, 1024)).copy()
    x[0, :32] = 1.0
    x[1, :32] = 0.0
    x[1, 32:64] = 448.0
    x[1, 96] = np.nextafter(np.float32(448.0), np.float32(1e9))
    x[1, 128:160] = np.float32(2.0 ** -149)
    x[2] *= np.float32(1e-30)
    x[3] *= np.float32(1e30)
    say("mx quantize vs C++")
    q, e = gpu_lib.mxfp8_quantize(to_dev(x))
    cq, ce = cpp_oracle.mx_quantize(x)
    assert np.array_equal(to_host(e), ce)
    assert np.array_equal(_codes(q), cq)


# (M, N, K) and the tiles they take on a 256-CU part: 64x128 (K tail), 128x128,
# 128x128 split over K, 256x128 (K tail), 256x256 (K tail), 256x256 with
# second tiles per workgroup
SHAPES_A = [(1000, 1001, 272), (1900, 2000, 1024), (512, 512, 8192), (2600, 2900, 1056), (2561, 3008, 272),
            (4000, 6400, 256)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", SHAPES_A)
def test_mode_a_matches_cpp(gpu_lib, M, N, K, out):
    import torch
    seed = M * 5 + N * 3 + K
    A, B = synth.u8_codes(seed, 1, (M, K)), synth.u8_codes(seed, 2, (N, K))
    sa, sb = _uscale(seed, M, 3), _uscale(seed, N, 4)
    say("mode a vs C++", M, N, K, out)
    D = gpu_lib.fp8_gemm_scaled(M, N, K, to_dev(A), to_dev(B), to_dev(sa), to_dev(sb),
                                out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    ref, W = cpp_oracle.gemm_scaled(A, B, sa, sb, weight=True)
    assert_gemm_close(to_host(D), ref, W, out, "mode a vs C++ %dx%dx%d %s" % (M, N, K, out),
                      alignment(A, B, sa, sb))


# 128x128 (whole scale dwords, a K tail of 32), 256x128 (K tail), 256x256, and
# 256x128 tiles of one stage, three per workgroup
SHAPES_B = [(257, 300, 4128), (2600, 2900, 1056), (2304, 4000, 1024), (4864, 4096, 128)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", SHAPES_B)
def test_mode_b_matches_cpp(gpu_lib, M, N, K, out):
    import torch
    seed = M * 7 + N * 5 + K
    A, B = synth.u8_codes(seed, 1, (M, K)), synth.u8_codes(seed, 2, (N, K))
    ea = (synth.u8_codes(seed, 7, (M, K // 32), exclude_nan=False) % 41 + 107).astype(np.uint8)
    eb = (synth.u8_codes(seed, 8, (N, K // 32), exclude_nan=False) % 41 + 107).astype(np.uint8)
    say("mode b vs C++", M, N, K, out)
    D = gpu_lib.mxfp8_gemm(M, N, K, to_dev(A), to_dev(B), to_dev(ea), to_dev(eb),
                           out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    ref, W = cpp_oracle.mxfp8_gemm(A, B, ea, eb, weight=True)
    assert_gemm_close(to_host(D), ref, W, out, "mode b vs C++ %dx%dx%d %s" % (M, N, K, out),
                      alignment(A, B, ea=ea, eb=eb))


def _full_size(gpu_lib, w, mx, fmt="e4m3"):
    """GPU quantize -> GPU GEMM at full size (bf16, the benchmark's launch, and
    fp32), against the C++ quantizers and the C++ GEMM.  fmt: both operands'
    format in mode (a) (E5M2: fp8_quantize_ex and fp8_gemm_scaled_ex, as the
    benchmark's --fmt-a e5m2 --fmt-b e5m2 step)."""
    import torch
    rows = band_rows(w.M)
    say("C++ full size", w.name, "draw")
    XA, XB = synth.draw(w, "a"), synth.draw(w, "b")
    say("C++ full size", w.name, "gpu")
    if mx:
        qa, sa = gpu_lib.mxfp8_quantize(to_dev(XA))
        qb, sb = gpu_lib.mxfp8_quantize(to_dev(XB))
        gemm_fn = gpu_lib.mxfp8_gemm
    elif fmt == "e5m2":
        F = gpu_lib.FMT_E5M2
        qa, sa = gpu_lib.fp8_quantize_ex(to_dev(XA), fmt=F)
        qb, sb = gpu_lib.fp8_quantize_ex(to_dev(XB), fmt=F)
        gemm_fn = lambda m, n, k, a, b, x, y, out_dtype: gpu_lib.fp8_gemm_scaled_ex(m, n, k, a, F, b, F, x, y,
                                                                                    out_dtype=out_dtype)
    else:
        qa, sa = gpu_lib.fp8_quantize_rowwise(to_dev(XA))
        qb, sb = gpu_lib.fp8_quantize_rowwise(to_dev(XB))
        gemm_fn = gpu_lib.fp8_gemm_scaled
    Ds = {}
    for out, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        D = gemm_fn(w.M, w.N, w.K, qa, qb, sa, sb, out_dtype=dt)
        torch.cuda.synchronize()
        Ds[out] = to_host(D[torch.from_numpy(rows).cuda()])
        del D
    say("C++ full size", w.name, "oracle")
    quantize = cpp_oracle.mx_quantize if mx else (lambda x: cpp_oracle.quantize_rowwise(x, fmt))
    oa, osa = quantize(XA[rows])
    ob, osb = quantize(XB)
    del XA, XB
    # the GPU's codes and scales are the C++ oracle's, bit for bit
    assert np.array_equal(_codes(qa)[rows], oa) and np.array_equal(_codes(qb), ob)
    sa_h, sb_h = to_host(sa), to_host(sb)
    if mx:
        assert np.array_equal(sa_h[rows], osa) and np.array_equal(sb_h, osb)
        ref, W = cpp_oracle.mxfp8_gemm(oa, ob, osa, osb, weight=True)
        T = alignment(oa, ob, ea=osa, eb=osb)
    else:
        assert np.array_equal(sa_h[rows].view(np.uint32), osa.view(np.uint32))
        assert np.array_equal(sb_h.view(np.uint32), osb.view(np.uint32))
        ref, W = cpp_oracle.gemm_scaled(oa, ob, osa, osb, fmt, fmt, weight=True)
        T = alignment(oa, ob, osa, osb, fmt_a=fmt, fmt_b=fmt)
    for out in ("bf16", "f32"):
        assert_gemm_close(Ds[out], ref, W, out, "%s %s vs C++ %s" % (w.name, fmt, out), T,
                          plain_max=PLAIN_MAX[(w.name, out)] if fmt == "e4m3" else PLAIN_MAX_E5M2[out])


def test_c3_matches_cpp(gpu_lib):
    _full_size(gpu_lib, synth.WORKLOADS["c3_8192x2048x8192"], mx=False)


def test_ffn_up_matches_cpp(gpu_lib):
    _full_size(gpu_lib, synth.WORKLOADS["c4_ffn_up_8192x22016x8192"], mx=False)


def test_ffn_up_e5m2_matches_cpp(gpu_lib):
    _full_size(gpu_lib, synth.WORKLOADS["c4_ffn_up_8192x22016x8192"], mx=False, fmt="e5m2")


def test_mx_workload_matches_cpp(gpu_lib):
    _full_size(gpu_lib, synth.WORKLOADS["c5_mx_4096x14336x4096"], mx=True)
