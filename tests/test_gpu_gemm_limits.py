"""GPU parity of the GEMMs at the largest sizes the library accepts.

The kernels address a 256-row panel of A, B (k bytes per row) or D (n elements
per row) with 32-bit offsets below 2^31, so the limits are k < 2^23 and
n < 2^22 (bf16 output) / 2^21 (fp32 output); the host rejects anything beyond.
Just inside each limit every output is checked: an offset that wrapped would
land in the wrong place of the panel.
"""

import numpy as np
import pytest

import synth
from gpu_util import alignment, assert_gemm_close, say, to_dev, to_host
from oracle import gemm

pytestmark = pytest.mark.gpu


def torch_dtype(out):
    import torch
    return torch.bfloat16 if out == "bf16" else torch.float32


@pytest.mark.parametrize("K", [(1 << 23) - 128, (1 << 23) - 16])
def test_mode_a_largest_k(gpu_lib, K):
    """k just below 2^23 (a whole number of 128-byte stages, and a K tail)."""
    M, N = 3, 5
    A = synth.u8_codes(0xB16, 1, (M, K))
    B = synth.u8_codes(0xB16, 2, (N, K))
    sa = np.array([0.5, 1.0, 2.0], np.float32)
    sb = np.array([1.0, 0.25, 4.0, 0.5, 1.5], np.float32)
    say("largest k", K)
    D = to_host(gpu_lib.fp8_gemm_scaled(M, N, K, to_dev(A), to_dev(B), to_dev(sa), to_dev(sb), out_dtype=torch_dtype("f32")))
    assert_gemm_close(D, gemm.gemm_scaled(A, B, sa, sb), gemm.gemm_scaled_weight(A, B, sa, sb), "f32",
                      "largest k %d" % K, alignment(A, B, sa, sb))


def test_mode_b_largest_k(gpu_lib):
    M, N, K = 2, 3, (1 << 23) - 128
    A = synth.u8_codes(0xB17, 1, (M, K))
    B = synth.u8_codes(0xB17, 2, (N, K))
    ea = (synth.u8_codes(0xB17, 3, (M, K // 32)) % 21 + 117).astype(np.uint8)
    eb = (synth.u8_codes(0xB17, 4, (N, K // 32)) % 21 + 117).astype(np.uint8)
    say("mx largest k", K)
    D = to_host(gpu_lib.mxfp8_gemm(M, N, K, to_dev(A), to_dev(B), to_dev(ea), to_dev(eb), out_dtype=torch_dtype("f32")))
    assert_gemm_close(D, gemm.mxfp8_gemm(A, B, ea, eb), gemm.mxfp8_gemm_weight(A, B, ea, eb), "f32",
                      "mx largest k", alignment(A, B, ea=ea, eb=eb))


@pytest.mark.parametrize("out,N", [("bf16", 1 << 22), ("f32", 1 << 21)])
def test_mode_a_largest_n(gpu_lib, out, N):
    """n at its limit for the output type: B repeats 97 distinct rows, so the
    oracle computes 97 columns and every output column must equal its row's."""
    import torch
    M, K, P = 300, 64, 97
    A = synth.u8_codes(0xB18, 1, (M, K))
    base = synth.u8_codes(0xB18, 2, (P, K))
    sa = (0.5 + synth.uniform(synth.stream_key(0xB18, 3), 0, M)).astype(np.float32)
    sb_base = (0.5 + synth.uniform(synth.stream_key(0xB18, 4), 0, P)).astype(np.float32)
    idx = torch.arange(N, device="cuda") % P
    Bd = to_dev(base)[idx].contiguous()
    sbd = to_dev(sb_base)[idx].contiguous()
    say("largest n", N, out)
    D = gpu_lib.fp8_gemm_scaled(M, N, K, to_dev(A), Bd, to_dev(sa), sbd, out_dtype=torch_dtype(out))
    ref = gemm.gemm_scaled(A, base, sa, sb_base)
    W = gemm.gemm_scaled_weight(A, base, sa, sb_base)
    T = alignment(A, base, sa, sb_base)
    # columns n and n + P*j must hold the same values: compare all N columns
    # against the P reference columns, P-column block by block on the device
    Dh = D.float().cpu().numpy().astype(np.float64) if out == "bf16" else D.cpu().numpy().astype(np.float64)
    full = N // P * P
    blocks = Dh[:, :full].reshape(M, N // P, P)
    assert_gemm_close(blocks[:, 0, :], ref, W, out, "largest n: first block", T)
    assert np.array_equal(blocks, np.broadcast_to(blocks[:, :1, :], blocks.shape)), "columns differ between blocks"
    assert_gemm_close(Dh[:, full:], ref[:, :N - full], W[:, :N - full], out, "largest n: tail", T[:, :N - full])
