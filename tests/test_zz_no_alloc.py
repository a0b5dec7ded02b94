"""fp8_gemm_scaled_noalloc, the GEMM entry point that allocates nothing (its
split workspace is a fixed device array in the library), against
fp8_gemm_scaled, through the C ABI.  Same kernels, so the outputs must agree
bit for bit.  Two calls in a row on shapes that split their tiles over K (the
array's counters must be back at zero after the first for the second to add
up the same), the second smaller; then a shape that does not split."""

import ctypes

import numpy as np
import pytest

import synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _codes(seed, shape, stream):
    return synth.u8_codes(seed, stream, shape)


def _call(lib, name, M, N, K, A, B, sa, sb, D, out):
    import torch
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = getattr(lib, name)(ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), P(A), P(B), P(sa), P(sb),
                            P(D), out, st)
    assert rc == 0, (name, rc)


# 512x512x8192: 16 tiles of 128, each split into 4 K ranges; 128x128x4096: one
# tile in 4; 1000x1001x272: no split (K tail; 64x128 tiles); 2600x2900x1024:
# 253 tiles of 256x128
@pytest.mark.parametrize("out", [0, 1])
def test_noalloc_matches_fp8_gemm_scaled(gpu_lib, out):
    import torch
    lib = gpu_lib.load()
    dt = torch.bfloat16 if out == 0 else torch.float32
    for M, N, K in ((512, 512, 8192), (128, 128, 4096), (1000, 1001, 272), (2600, 2900, 1024)):
        seed = 7 * M + N + K
        A, B = to_dev(_codes(seed, (M, K), 1)), to_dev(_codes(seed, (N, K), 2))
        sa = to_dev((0.5 + synth.uniform(synth.stream_key(seed, 3), 0, M)).astype(np.float32))
        sb = to_dev((0.5 + synth.uniform(synth.stream_key(seed, 4), 0, N)).astype(np.float32))
        D0 = torch.full((M, N), 7.0, dtype=dt, device="cuda")
        D1 = torch.full((M, N), -7.0, dtype=dt, device="cuda")
        say("noalloc vs fp8_gemm_scaled", M, N, K, out)
        _call(lib, "fp8_gemm_scaled", M, N, K, A, B, sa, sb, D0, out)
        _call(lib, "fp8_gemm_scaled_noalloc", M, N, K, A, B, sa, sb, D1, out)
        torch.cuda.synchronize()
        iv = torch.int16 if out == 0 else torch.int32
        assert torch.equal(D0.view(iv), D1.view(iv)), (M, N, K, out)
