"""The two scaled-GEMM definitions in float64 -- oracle, test infrastructure.

Mode (a), per-token x per-channel scales:
    D[m,n] = sa[m] * sb[n] * sum_k dec(A[m,k]) * dec(B[n,k])
A is [M,K] (tokens x hidden), B is [N,K] (output channels x hidden), both with
K contiguous.  Source: the DeepGEMM call on the page
"FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM" (GEMM-call example: m = tokens,
n, k = hidden, ``scale_a`` one fp32 per token, ``scale_b`` one fp32 per
channel) and the shapes of its ``benchmark_gemm`` runs.

The float64 sum is exact: every decoded value is an integer multiple of 2^-9
below 2^9, so each product is a multiple of 2^-18 below 2^18, and any sum of
fewer than 2^35 of them is a multiple of 2^-18 below 2^53.  Hence any
summation order (a BLAS matmul included) gives the same float64 value.

Mode (b), MXFP8 block scales (one UE8M0 code per 32 consecutive K elements of
each row of A and of B; page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합",
sections 1 and 2):
    D[m,n] = sum_j 2^(ea[m,j]-127) * 2^(eb[n,j]-127)
                   * sum_{t<32} dec(A[m,32j+t]) * dec(B[n,32j+t])
Each block sum is exact; the sum over blocks rounds in float64 only.

Operand formats: each of A and B is E4M3 (the default) or E5M2 (oracle.e5m2),
as the matrix-core instruction takes a format per operand.  With an E5M2
operand the products span up to 2^-32 .. 2^32 and the float64 sum is no
longer exact: it is the definition rounded in float64, within
K * 2^-53 * W of it (the standard bound for a sum of K terms), which is below
2^-30 W for every K this library takes (k < 2^23) -- five orders of magnitude
inside the 1e-5 W term of the bound below.

Error bound for a GPU result accumulated in fp32 (stated for this library):
    |D_gpu - D_ref| <= 1e-5 * W + ulp_out(D_ref) + T
with W = |sa*sb| * sum_k |dec(A) dec(B)| (mode a) or the same sum with the
block scale factors (mode b), and ulp_out the spacing of the output format
at D_ref (bf16: 2^(max(floor(log2|x|),-126)-7), 2^-133 at zero; fp32: -23
and 2^-149).  The first two terms are the fp32-accumulation bound; T is the
matrix-core truncation term below.  The first two terms alone ("the plain
bound") are the bound the products would meet if the matrix core summed
them exactly; the gfx950 FP8 matrix core does not.

Matrix-core truncation term T.  Measured on MI355X for every gfx950 FP8
matrix-core instruction (the scaled 32x32x64 and 16x16x128 forms and the
older 32x32x16 and 16x16x32 ones): each run of 8 consecutive K products is
added in fixed point aligned to the run's largest exponent sum
E = max(x_a + x_b) (x: the unbiased exponent field, zeros and subnormals at
the smallest normal exponent), keeping 13 bits below 2^E; each product's
bits below 2^(E-13) are dropped (truncation toward zero).  (1024 + 2^-8 in one
run gives 1024, in two runs 1024.00390625; 2^10 + 3*2^-4 gives 1024.125;
4 + 2^-12 gives 4 while 1.875^2 + 2^-13 is exact, so E is the exponent sum,
not the product's exponent.)  The runs' sums and the accumulator are then
combined with about 24 bits kept below the larger operand and rounded to
fp32: a few fp32 ulps of the instruction's result at most, inside the
fp32-accumulation terms.  A product is an integer multiple of
2^(x_a - mant_a + x_b - mant_b), so it is exact when that step is at least
the run's grid 2^(E-13); otherwise it loses less than the grid and at most
its own magnitude.  Hence, per output element,
    T[m,n] = |sa sb| * sum_runs sum_{t: p_t off the grid} min(|p_t|, 2^(E_run - 13))
(mode b: each run's sum times the scale factors of its 32-element block).
For N(0,1)-like operands T is far below 1e-5 * W; for operands whose runs
mix magnitudes 2^13 apart (uniform random codes, x50 outliers) it is not.
"""

import numpy as np

from . import e4m3, e5m2
from .quant import MX_BLOCK, ue8m0_value

REL_TOL = 1e-5
MFMA_GROUP = 8          # consecutive K products the matrix core aligns together (a "run")
MFMA_KEEP_BITS = 13     # bits kept below the run's largest exponent sum


FORMATS = {"e4m3": e4m3, "e5m2": e5m2}


def _decoded(codes, fmt="e4m3"):
    d = FORMATS[fmt].decode(codes)
    if not np.isfinite(d).all():
        raise ValueError("%s NaN or infinity code in a GEMM operand" % fmt)
    return d


def gemm_scaled(A, B, sa, sb, fmt_a="e4m3", fmt_b="e4m3") -> np.ndarray:
    """Mode (a) result in float64 [M,N]."""
    Ad, Bd = _decoded(A, fmt_a), _decoded(B, fmt_b)
    S = Ad @ Bd.T                                   # exact for E4M3 (see module docstring)
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    return S * sa[:, None] * sb[None, :]


def gemm_scaled_weight(A, B, sa, sb, fmt_a="e4m3", fmt_b="e4m3") -> np.ndarray:
    """W[m,n] = |sa[m] sb[n]| * sum_k |dec(A[m,k]) dec(B[n,k])| (float64)."""
    Ad, Bd = np.abs(_decoded(A, fmt_a)), np.abs(_decoded(B, fmt_b))
    sa = np.abs(np.asarray(sa, dtype=np.float32).astype(np.float64))
    sb = np.abs(np.asarray(sb, dtype=np.float32).astype(np.float64))
    return (Ad @ Bd.T) * sa[:, None] * sb[None, :]


def _mx_terms(A, B, ea, eb, absolute, fmt_a, fmt_b):
    Ad, Bd = _decoded(A, fmt_a), _decoded(B, fmt_b)
    if absolute:
        Ad, Bd = np.abs(Ad), np.abs(Bd)
    M, K = Ad.shape
    N = Bd.shape[0]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32 for MX blocks")
    nb = K // MX_BLOCK
    ea = np.asarray(ea).reshape(M, nb)
    eb = np.asarray(eb).reshape(N, nb)
    D = np.zeros((M, N), dtype=np.float64)
    for j in range(nb):
        blk = slice(MX_BLOCK * j, MX_BLOCK * (j + 1))
        Sj = Ad[:, blk] @ Bd[:, blk].T                       # exact block sum
        D += ue8m0_value(ea[:, j])[:, None] * ue8m0_value(eb[:, j])[None, :] * Sj
    return D


def mxfp8_gemm(A, B, ea, eb, fmt_a="e4m3", fmt_b="e4m3") -> np.ndarray:
    """Mode (b) result in float64 [M,N]."""
    return _mx_terms(A, B, ea, eb, False, fmt_a, fmt_b)


def mxfp8_gemm_weight(A, B, ea, eb, fmt_a="e4m3", fmt_b="e4m3") -> np.ndarray:
    """Error-bound weight for mode (b): the same sum over |products|."""
    return _mx_terms(A, B, ea, eb, True, fmt_a, fmt_b)


# exponent field (shift, mask) and bias of each operand format
_EXP_FIELD = {"e4m3": (3, 0xF, 7), "e5m2": (2, 0x1F, 15)}


def code_exponent(codes, fmt="e4m3") -> np.ndarray:
    """Alignment exponent of codes: the unbiased exponent field, with
    subnormals and zeros at the smallest normal exponent (exponent field 0
    read as 1): -6 for E4M3, -14 for E5M2."""
    shift, mask, bias = _EXP_FIELD[fmt]
    c = np.asarray(codes, dtype=np.uint8)
    e = (c >> shift) & mask
    return np.maximum(e, 1).astype(np.int64) - bias


def alignment_term(A, B, sa=None, sb=None, ea=None, eb=None, fmt_a="e4m3", fmt_b="e4m3") -> np.ndarray:
    """T[m,n]: bound of the matrix core's in-run truncation (module docstring),
    computed per output element from its own products.

    Mode (a): pass sa, sb (fp32 per row); mode (b): pass ea, eb (UE8M0 codes
    per 32-block); neither: unscaled.  A ragged last run of K is padded with
    zero codes, as the hardware sees them.  One row of A at a time; for
    full-size checks oracle.cpp_oracle.alignment_term computes the same
    definition in a threaded loop.
    """
    Ad, Bd = np.abs(_decoded(A, fmt_a)), np.abs(_decoded(B, fmt_b))
    xa, xb = code_exponent(A, fmt_a), code_exponent(B, fmt_b)
    M, K = Ad.shape
    N = Bd.shape[0]
    G = -(-K // MFMA_GROUP)

    def runs(v, x, fmt):
        R = v.shape[0]
        vp = np.zeros((R, G * MFMA_GROUP), np.float64)
        xp = np.full((R, G * MFMA_GROUP), 1 - _EXP_FIELD[fmt][2], np.int64)   # zero codes
        vp[:, :K], xp[:, :K] = v, x
        return vp.reshape(R, G, MFMA_GROUP), xp.reshape(R, G, MFMA_GROUP)

    Av, Ax = runs(Ad, xa, fmt_a)
    Bv, Bx = runs(Bd, xb, fmt_b)
    if ea is not None:
        per = 32 // MFMA_GROUP
        fa = np.repeat(ue8m0_value(np.asarray(ea).reshape(M, -1)), per, axis=1)[:, :G]
        fb = np.repeat(ue8m0_value(np.asarray(eb).reshape(N, -1)), per, axis=1)[:, :G]
    T = np.zeros((M, N), np.float64)
    for m in range(M):
        E = (Ax[m][None, :, :] + Bx).max(axis=2)                   # [N, G] largest exponent sum of each run
        grid = np.ldexp(1.0, E - MFMA_KEEP_BITS)[:, :, None]
        p = Av[m][None, :, :] * Bv                                   # [N, G, 8] |products|, exact
        q = p / grid                                                 # exact: the grid is a power of two
        run = np.where(q != np.floor(q), np.minimum(p, grid), 0.0).sum(axis=2)
        if ea is not None:
            run = run * fa[m][None, :] * fb
        T[m] = run.sum(axis=1)
    if sa is not None:
        sa = np.abs(np.asarray(sa, dtype=np.float32).astype(np.float64))
        sb = np.abs(np.asarray(sb, dtype=np.float32).astype(np.float64))
        T = T * sa[:, None] * sb[None, :]
    return T


def ulp(x, out_dtype: str) -> np.ndarray:
    """Spacing of bf16 or fp32 at x (float64 array), subnormal floor included."""
    mant_bits = {"bf16": 7, "f32": 23}[out_dtype]
    x = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    # log2 of a float64 can misround just below a power of two; fix it exactly.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > x, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= x, e + 1, e)
    e = np.maximum(e, -126)
    return np.where(x > 0, np.ldexp(1.0, (e - mant_bits).astype(np.int64)),
                    np.ldexp(1.0, -126 - mant_bits))


def tolerance(D_ref, W, out_dtype: str, T=None) -> np.ndarray:
    tol = REL_TOL * np.asarray(W, dtype=np.float64) + ulp(D_ref, out_dtype)
    return tol if T is None else tol + T


def check(D_gpu, D_ref, W, out_dtype: str, T=None):
    """Element-by-element comparison against the bound (with the alignment
    term T if given).

    Returns (ok, worst error/tolerance ratio, number of elements over the bound).
    """
    D_gpu = np.asarray(D_gpu, dtype=np.float64)
    err = np.abs(D_gpu - D_ref)
    tol = tolerance(D_ref, W, out_dtype, T)
    bad = ~(err <= tol)                 # NaN in D_gpu counts as a failure
    ratio = float(np.max(np.where(np.isnan(err), np.inf, err / tol))) if err.size else 0.0
    return (not bad.any()), ratio, int(bad.sum())
