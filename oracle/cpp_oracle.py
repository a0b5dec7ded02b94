"""ctypes access to the plain C++ oracle (oracle/cpp/fp8_oracle.cpp) -- test
infrastructure, like the rest of oracle/.

The C++ oracle restates the numpy oracle's definitions in scalar C++ (FP8
decode from the bit fields, the saturating round-to-nearest-even cast written
twice -- as the nearest decoded magnitude and as integer bit manipulation --,
the row-wise and MX block quantizers, both GEMM modes in double with the
error bound's weight, and the matrix-core truncation term of
oracle.gemm.alignment_term).  Tests use it to check the cast on every fp32 bit
pattern, to check the two oracles against each other, and as the reference
of GPU results (tests/test_gpu_cpp_oracle.py).  The heavy loops split rows or
output columns over host threads (`threads`; 0: OMP_NUM_THREADS if set, else
the CPU count, at most 16); each output is still one sequential loop, so the
results do not depend on the thread count.  build() compiles it with g++
(host only).
"""

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "fp8_oracle.cpp")
LIB = os.path.join(HERE, "cpp", "libfp8_oracle.so")
FMT = {"e4m3": 0, "e5m2": 1}

_lib = None


def build() -> str:
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("no host C++ compiler (g++) for the C++ oracle")
    tmp = LIB + ".tmp"
    res = subprocess.run([cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-o", tmp, SRC], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C++ oracle failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P, I64, U8, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint8, ctypes.c_int
        lib.fp8o_decode.argtypes, lib.fp8o_decode.restype = [I, U8], ctypes.c_double
        lib.fp8o_encode_nearest.argtypes, lib.fp8o_encode_nearest.restype = [I, ctypes.c_float], U8
        lib.fp8o_encode_bits.argtypes, lib.fp8o_encode_bits.restype = [I, ctypes.c_float], U8
        lib.fp8o_cast_sweep.argtypes, lib.fp8o_cast_sweep.restype = [I, ctypes.c_uint64, ctypes.c_uint64, P], I64
        lib.fp8o_encode_array.argtypes, lib.fp8o_encode_array.restype = [I, P, I64, P], None
        lib.fp8o_quantize_rowwise.argtypes, lib.fp8o_quantize_rowwise.restype = [I, P, I64, I64, P, P, I], None
        lib.fp8o_mx_quantize.argtypes, lib.fp8o_mx_quantize.restype = [P, I64, I64, P, P, I], None
        lib.fp8o_gemm_scaled.argtypes, lib.fp8o_gemm_scaled.restype = [I, I, I64, I64, I64, P, P, P, P, P, P, I], None
        lib.fp8o_gemm_mx.argtypes, lib.fp8o_gemm_mx.restype = [I, I, I64, I64, I64, P, P, P, P, P, P, I], None
        lib.fp8o_alignment_term.argtypes = [I, I, I64, I64, I64, P, P, P, P, P, I]
        lib.fp8o_alignment_term.restype = None
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _threads(threads):
    if threads > 0:
        return int(threads)
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return min(n, 16)


def decode_table(fmt="e4m3"):
    lib = load()
    return np.array([lib.fp8o_decode(FMT[fmt], c) for c in range(256)], dtype=np.float64)


def cast_sweep(lo, hi, fmt="e4m3"):
    """(number of fp32 patterns in [lo, hi) where the two casts differ, first such pattern or None)."""
    first = ctypes.c_uint32(0)
    bad = load().fp8o_cast_sweep(FMT[fmt], lo, hi, ctypes.byref(first))
    return bad, (first.value if bad else None)


def encode(x, fmt="e4m3"):
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape, np.uint8)
    load().fp8o_encode_array(FMT[fmt], _p(x), x.size, _p(q))
    return q


def quantize_rowwise(x, fmt="e4m3", threads=0):
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(R, np.float32)
    load().fp8o_quantize_rowwise(FMT[fmt], _p(x), R, C, _p(q), _p(s), _threads(threads))
    return q, s


def mx_quantize(x, threads=0):
    """MX block quantization of fp32 rows (row length a multiple of 32, finite
    values): (E4M3 codes [R, C], UE8M0 scale codes [R, C/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    if C % 32:
        raise ValueError("MX blocks need the row length to be a multiple of 32")
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, C // 32), np.uint8)
    load().fp8o_mx_quantize(_p(x), R, C, _p(q), _p(e), _threads(threads))
    return q, e


def gemm_scaled(A, B, sa, sb, fmt_a="e4m3", fmt_b="e4m3", weight=False, threads=0):
    """Mode (a) in double, [M, N]; with weight=True also the error bound's W."""
    A, B = np.ascontiguousarray(A, np.uint8), np.ascontiguousarray(B, np.uint8)
    sa, sb = np.ascontiguousarray(sa, np.float32), np.ascontiguousarray(sb, np.float32)
    M, K = A.shape
    N = B.shape[0]
    D = np.empty((M, N), np.float64)
    W = np.empty((M, N), np.float64) if weight else None
    load().fp8o_gemm_scaled(FMT[fmt_a], FMT[fmt_b], M, N, K, _p(A), _p(B), _p(sa), _p(sb), _p(D),
                            _p(W) if weight else None, _threads(threads))
    return (D, W) if weight else D


def mxfp8_gemm(A, B, ea, eb, fmt_a="e4m3", fmt_b="e4m3", weight=False, threads=0):
    """Mode (b) in double, [M, N]; with weight=True also the error bound's W."""
    A, B = np.ascontiguousarray(A, np.uint8), np.ascontiguousarray(B, np.uint8)
    ea, eb = np.ascontiguousarray(ea, np.uint8), np.ascontiguousarray(eb, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    D = np.empty((M, N), np.float64)
    W = np.empty((M, N), np.float64) if weight else None
    load().fp8o_gemm_mx(FMT[fmt_a], FMT[fmt_b], M, N, K, _p(A), _p(B), _p(ea), _p(eb), _p(D),
                        _p(W) if weight else None, _threads(threads))
    return (D, W) if weight else D


def alignment_term(A, B, sa=None, sb=None, ea=None, eb=None, fmt_a="e4m3", fmt_b="e4m3", threads=0):
    """The matrix-core truncation term T (oracle.gemm.alignment_term's
    definition), computed by the threaded C++ loop: same arguments."""
    A, B = np.ascontiguousarray(A, np.uint8), np.ascontiguousarray(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    for codes, fmt in ((A, fmt_a), (B, fmt_b)):
        if not np.isfinite(decode_table(fmt)[codes & 0x7F]).all():
            raise ValueError("%s NaN or infinity code in a GEMM operand" % fmt)
    T = np.empty((M, N), np.float64)
    if ea is not None:
        ea = np.ascontiguousarray(ea, np.uint8)
        eb = np.ascontiguousarray(eb, np.uint8)
        load().fp8o_alignment_term(FMT[fmt_a], FMT[fmt_b], M, N, K, _p(A), _p(B), _p(ea), _p(eb), _p(T),
                                   _threads(threads))
    else:
        load().fp8o_alignment_term(FMT[fmt_a], FMT[fmt_b], M, N, K, _p(A), _p(B), None, None, _p(T),
                                   _threads(threads))
    if sa is not None:
        sa = np.abs(np.asarray(sa, dtype=np.float32).astype(np.float64))
        sb = np.abs(np.asarray(sb, dtype=np.float32).astype(np.float64))
        T = T * sa[:, None] * sb[None, :]
    return T
