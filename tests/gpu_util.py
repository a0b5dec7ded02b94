"""Helpers for the GPU parity tests: upload seeded inputs, run the oracle on
row chunks, compare element by element.  Test infrastructure only."""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import cpp_oracle, e4m3, gemm, quant  # noqa: E402


def say(*args):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *args, flush=True)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def oracle_quantize_rows(x, chunk=256):
    """The oracle's row-wise quantizer, a block of rows at a time (row-local, so exact)."""
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(R, np.float32)
    for r in range(0, R, chunk):
        q[r:r + chunk], s[r:r + chunk] = quant.quantize_rowwise(x[r:r + chunk])
    return q, s


def oracle_cast(x, chunk=1 << 18):
    flat = np.ascontiguousarray(x).reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    for i in range(0, flat.size, chunk):
        out[i:i + chunk] = e4m3.encode(flat[i:i + chunk])
    return out.reshape(x.shape)


def alignment(A, B, sa=None, sb=None, ea=None, eb=None, fmt_a="e4m3", fmt_b="e4m3"):
    """The matrix-core truncation term T of the bound: the numpy definition
    (oracle.gemm.alignment_term) for small problems, the threaded C++ loop of
    the same definition (oracle.cpp_oracle.alignment_term) for large ones."""
    M, K = np.shape(A)
    N = np.shape(B)[0]
    if M * N * K <= (1 << 24):
        return gemm.alignment_term(A, B, sa, sb, ea, eb, fmt_a, fmt_b)
    return cpp_oracle.alignment_term(A, B, sa, sb, ea, eb, fmt_a, fmt_b)


def assert_gemm_close(D_gpu, D_ref, W, out, what="", T=None, plain_max=None):
    """Element-by-element check against the bound 1e-5 W + ulp + T (T: the
    matrix-core truncation term).  Also counts the elements over the plain
    fp32-accumulation bound 1e-5 W + ulp (T = 0) and, when plain_max is given,
    asserts that count is at most plain_max.  Returns (worst error / tolerance
    with T, elements over the plain bound)."""
    ok, ratio, nbad = gemm.check(D_gpu, D_ref, W, out, T)
    _, plain_ratio, plain_bad = gemm.check(D_gpu, D_ref, W, out)
    say("%s: worst err/tol %.3g (plain bound: %.3g); plain 1e-5 bound met by %d of %d"
        % (what, ratio, plain_ratio, D_ref.size - plain_bad, D_ref.size))
    if not ok:
        err = np.abs(np.asarray(D_gpu, np.float64) - D_ref)
        tol = gemm.tolerance(D_ref, W, out, T)
        idx = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err / tol)), err.shape)
        raise AssertionError("%s: %d of %d elements over the bound; worst at %s: gpu %r ref %r tol %r"
                             % (what, nbad, err.size, idx, D_gpu[idx], D_ref[idx], tol[idx]))
    if plain_max is not None:
        assert plain_bad <= plain_max, ("%s: %d elements over the plain bound, more than the %d recorded for "
                                        "these kernels" % (what, plain_bad, plain_max))
    return ratio, plain_bad


def oracle_mx_rows(x, chunk=256):
    """The oracle's MX block quantizer, a block of rows at a time (row-local, so exact)."""
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, C // 32), np.uint8)
    for r in range(0, R, chunk):
        q[r:r + chunk], e[r:r + chunk] = quant.mx_quantize(x[r:r + chunk])
    return q, e
