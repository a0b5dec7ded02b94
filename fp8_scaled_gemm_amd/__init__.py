"""fp8g -- FP8 scaled GEMM and quantizers for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/fp8g.h`` (libfp8g.so, built
in-tree by ``python -m fp8_scaled_gemm_amd.build``).  Every computation runs in
the library's HIP kernels; this module only checks tensors, allocates outputs
with torch, and passes raw device pointers and torch's current HIP stream.
There is no fallback: if the library is missing, every call raises.

Functions keep the C names and argument order:

    fp8_quantize_rowwise(x)                              -> (q, scale)
    fp8_quantize_ex(x, per_tensor=False, fmt=FMT_E4M3)   -> (q, scale)  (fp32 or bf16 x)
    mxfp8_quantize(x)                                    -> (q, scale codes)
    fp8_gemm_scaled(m, n, k, A, B, scale_a, scale_b)     -> D
    fp8_gemm_scaled_noalloc(m, n, k, A, B, scale_a, scale_b, D)  (D given: the
                                            library allocates nothing)
    mxfp8_gemm(m, n, k, A, B, scale_a, scale_b)          -> D
    fp8_gemm_scaled_ex(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b)  -> D
    mxfp8_gemm_ex(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b)       -> D
                                            (fmt: FMT_E4M3 or FMT_E5M2 per operand)
    concat_mla_k(k_nope, k_rope)                         -> k  (MLA key rows)
    fp8g_roof_mfma(blocks, iters), fp8g_roof_stream(src, dst, write_ratio)
                                            (roof probes for the benchmark)

E4M3 tensors are ``torch.float8_e4m3fn`` (OCP, the gfx950 format) and E5M2
tensors ``torch.float8_e5m2``, or either as raw ``torch.uint8`` codes; the
FNUZ variants of gfx942 are rejected.
"""

import ctypes
import os
import re

__all__ = ["load", "fp8_quantize_rowwise", "fp8_quantize_ex", "mxfp8_quantize", "fp8_gemm_scaled",
           "fp8_gemm_scaled_noalloc", "mxfp8_gemm",
           "fp8_gemm_scaled_ex", "mxfp8_gemm_ex", "concat_mla_k", "fp8g_roof_mfma", "fp8g_roof_stream",
           "status_string",
           "Fp8gError", "LIB_PATH", "HEADER_PATH", "OUT_BF16", "OUT_F32", "FMT_E4M3", "FMT_E5M2"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8g.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp8g.h")
OUT_BF16, OUT_F32 = 0, 1
FMT_E4M3, FMT_E5M2 = 0, 1

_lib = None

_VOIDP = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = {
    "fp8_quantize_rowwise": [_VOIDP, _I64, _I64, _VOIDP, _VOIDP, _VOIDP],
    "mxfp8_quantize": [_VOIDP, _I64, _I64, _VOIDP, _VOIDP, _VOIDP],
    "fp8_quantize_ex": [_VOIDP, ctypes.c_int, _I64, _I64, ctypes.c_int, ctypes.c_int, _VOIDP, _VOIDP, _VOIDP],
    "fp8_gemm_scaled": [_I64, _I64, _I64, _VOIDP, _VOIDP, _VOIDP, _VOIDP, _VOIDP, ctypes.c_int, _VOIDP],
    "fp8_gemm_scaled_noalloc": [_I64, _I64, _I64, _VOIDP, _VOIDP, _VOIDP, _VOIDP, _VOIDP, ctypes.c_int, _VOIDP],
    "mxfp8_gemm": [_I64, _I64, _I64, _VOIDP, _VOIDP, _VOIDP, _VOIDP, _VOIDP, ctypes.c_int, _VOIDP],
    "fp8_gemm_scaled_ex": [_I64, _I64, _I64, _VOIDP, ctypes.c_int, _VOIDP, ctypes.c_int, _VOIDP, _VOIDP, _VOIDP,
                           ctypes.c_int, _VOIDP],
    "mxfp8_gemm_ex": [_I64, _I64, _I64, _VOIDP, ctypes.c_int, _VOIDP, ctypes.c_int, _VOIDP, _VOIDP, _VOIDP,
                      ctypes.c_int, _VOIDP],
    "concat_mla_k": [_VOIDP, _VOIDP, _VOIDP, _I64, _I64, _I64, ctypes.c_int, _VOIDP],
    "fp8g_gemm_schedule": [_I64, _I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)],
    "fp8g_roof_mfma": [_I64, _I64, _VOIDP, _VOIDP],
    "fp8g_roof_stream": [_VOIDP, _I64, _VOIDP, ctypes.c_int, ctypes.c_int, _VOIDP],
}


class Fp8gError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: status %d (%s)" % (where, status, status_string(status)))


def header_functions():
    """Names of the functions declared in include/fp8g.h."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def load():
    """Load libfp8g.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp8g.so is not built; run `python -m fp8_scaled_gemm_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.fp8g_status_string.argtypes = [ctypes.c_int]
        lib.fp8g_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().fp8g_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise Fp8gError(status, where)


# ----------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _as_codes(t, name, fmt=FMT_E4M3):
    """uint8 view of an operand of format fmt (its float8 dtype or raw codes)."""
    torch = _torch()
    want = {FMT_E4M3: torch.float8_e4m3fn, FMT_E5M2: torch.float8_e5m2}.get(fmt)
    if want is None:
        raise ValueError("%s: format must be FMT_E4M3 or FMT_E5M2, got %r" % (name, fmt))
    if t.dtype == want:
        return t.view(torch.uint8)
    if t.dtype == torch.uint8:
        return t
    if t.dtype in (getattr(torch, "float8_e4m3fnuz", None), getattr(torch, "float8_e5m2fnuz", None)):
        raise TypeError("%s: %s (gfx942) is not an OCP format used on gfx950" % (name, t.dtype))
    raise TypeError("%s must be %s or uint8 codes, got %s" % (name, want, t.dtype))


def _need(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    cur = _torch().cuda.current_device()
    if t.device.index != cur:
        # the kernels run on the current device and take raw pointers
        raise ValueError("%s is on %s but the current device is cuda:%d (call under torch.cuda.device(%s))"
                         % (name, t.device, cur, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _out_code(out_dtype):
    torch = _torch()
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    if out_dtype == torch.float32:
        return OUT_F32
    raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")


def fp8_quantize_rowwise(x, q=None, scale=None):
    """Per-row E4M3 quantization of a 2-D fp32 device tensor.

    Returns (q: float8_e4m3fn [R, C], scale: float32 [R]) with x ~ q * scale.
    ``q`` and ``scale`` may be passed in (uint8 or float8_e4m3fn / float32).
    """
    torch = _torch()
    _need(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.float8_e4m3fn, device=x.device)
    if scale is None:
        scale = torch.empty((R,), dtype=torch.float32, device=x.device)
    qc = _as_codes(q, "q")
    _need(qc, "q", shape=(R, C))
    _need(scale, "scale", torch.float32, (R,))
    _check(load().fp8_quantize_rowwise(_ptr(x), R, C, _ptr(qc), _ptr(scale), _stream()),
           "fp8_quantize_rowwise")
    return q, scale


IN_F32, IN_BF16 = 0, 1
SCALE_PER_ROW, SCALE_PER_TENSOR = 0, 1


def fp8_quantize_ex(x, per_tensor=False, q=None, scale=None, fmt=FMT_E4M3):
    """FP8 quantization of a 2-D fp32 or bf16 device tensor with scale
    amax / MAX (448 for FMT_E4M3, 57344 for FMT_E5M2), one per row (scale [R])
    or one per tensor (scale [1]).  q is float8_e4m3fn or float8_e5m2."""
    torch = _torch()
    if x.dtype == torch.float32:
        code = IN_F32
    elif x.dtype == torch.bfloat16:
        code = IN_BF16
    else:
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    _need(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if q is None:
        qdt = {FMT_E4M3: torch.float8_e4m3fn, FMT_E5M2: torch.float8_e5m2}.get(fmt)
        if qdt is None:
            raise ValueError("fmt must be FMT_E4M3 or FMT_E5M2, got %r" % (fmt,))
        q = torch.empty((R, C), dtype=qdt, device=x.device)
    if scale is None:
        scale = torch.empty((1 if per_tensor else R,), dtype=torch.float32, device=x.device)
    qc = _as_codes(q, "q", fmt)
    _need(qc, "q", shape=(R, C))
    _need(scale, "scale", torch.float32, (1 if per_tensor else R,))
    _check(load().fp8_quantize_ex(_ptr(x), code, R, C, SCALE_PER_TENSOR if per_tensor else SCALE_PER_ROW, fmt,
                                  _ptr(qc), _ptr(scale), _stream()), "fp8_quantize_ex")
    return q, scale


def mxfp8_quantize(x, q=None, scale=None):
    """MXFP8 block quantization of a 2-D fp32 device tensor (cols % 32 == 0).

    Returns (q: float8_e4m3fn [R, C], scale: uint8 UE8M0 codes [R, C/32]) with
    x ~ q * 2^(scale - 127) per block of 32 along a row.
    """
    torch = _torch()
    _need(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if C % 32:
        raise ValueError("the row length must be a multiple of 32 for MXFP8")
    if q is None:
        q = torch.empty((R, C), dtype=torch.float8_e4m3fn, device=x.device)
    if scale is None:
        scale = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    qc = _as_codes(q, "q")
    _need(qc, "q", shape=(R, C))
    _need(scale, "scale", torch.uint8, (R, C // 32))
    _check(load().mxfp8_quantize(_ptr(x), R, C, _ptr(qc), _ptr(scale), _stream()), "mxfp8_quantize")
    return q, scale


def _gemm_operands(m, n, k, A, B, fmt_a=FMT_E4M3, fmt_b=FMT_E4M3):
    Ac, Bc = _as_codes(A, "A", fmt_a), _as_codes(B, "B", fmt_b)
    _need(Ac, "A", shape=(m, k))
    _need(Bc, "B", shape=(n, k))
    return Ac, Bc


def _out(m, n, A, D, out_dtype):
    torch = _torch()
    code = _out_code(out_dtype)
    if D is None:
        D = torch.empty((m, n), dtype=out_dtype, device=A.device)
    _need(D, "D", out_dtype, (m, n))
    return D, code


def fp8_gemm_scaled_ex(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b, D=None, out_dtype=None):
    """D[m,n] = scale_a[m] * scale_b[n] * sum_k A[m,k] * B[n,k] with A of format
    fmt_a and B of format fmt_b (FMT_E4M3 / FMT_E5M2)."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    Ac, Bc = _gemm_operands(m, n, k, A, B, fmt_a, fmt_b)
    _need(scale_a, "scale_a", torch.float32, (m,))
    _need(scale_b, "scale_b", torch.float32, (n,))
    D, code = _out(m, n, A, D, out_dtype)
    _check(load().fp8_gemm_scaled_ex(m, n, k, _ptr(Ac), fmt_a, _ptr(Bc), fmt_b, _ptr(scale_a), _ptr(scale_b),
                                     _ptr(D), code, _stream()), "fp8_gemm_scaled_ex")
    return D


def fp8_gemm_scaled(m, n, k, A, B, scale_a, scale_b, D=None, out_dtype=None):
    """D[m,n] = scale_a[m] * scale_b[n] * sum_k A[m,k] * B[n,k] (A [m,k], B [n,k], E4M3)."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    Ac, Bc = _gemm_operands(m, n, k, A, B)
    _need(scale_a, "scale_a", torch.float32, (m,))
    _need(scale_b, "scale_b", torch.float32, (n,))
    D, code = _out(m, n, A, D, out_dtype)
    _check(load().fp8_gemm_scaled(m, n, k, _ptr(Ac), _ptr(Bc), _ptr(scale_a), _ptr(scale_b), _ptr(D),
                                  code, _stream()), "fp8_gemm_scaled")
    return D


def fp8_gemm_scaled_noalloc(m, n, k, A, B, scale_a, scale_b, D, out_dtype=None):
    """fp8_gemm_scaled with the library's fixed split workspace: the C call
    allocates nothing.  D (the output, [m, n] of out_dtype, default bf16) must
    be given, so that this binding allocates nothing either."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if D is None:
        raise ValueError("fp8_gemm_scaled_noalloc: pass D (the output), the call allocates nothing")
    Ac, Bc = _gemm_operands(m, n, k, A, B)
    _need(scale_a, "scale_a", torch.float32, (m,))
    _need(scale_b, "scale_b", torch.float32, (n,))
    D, code = _out(m, n, A, D, out_dtype)
    _check(load().fp8_gemm_scaled_noalloc(m, n, k, _ptr(Ac), _ptr(Bc), _ptr(scale_a), _ptr(scale_b), _ptr(D),
                                          code, _stream()), "fp8_gemm_scaled_noalloc")
    return D


def _mx_scales(m, n, k, scale_a, scale_b):
    torch = _torch()
    if k % 32:
        raise ValueError("k must be a multiple of 32 for MXFP8")
    _need(scale_a, "scale_a", torch.uint8, (m, k // 32))
    _need(scale_b, "scale_b", torch.uint8, (n, k // 32))


def mxfp8_gemm_ex(m, n, k, A, fmt_a, B, fmt_b, scale_a, scale_b, D=None, out_dtype=None):
    """MX GEMM with A of format fmt_a and B of format fmt_b (FMT_E4M3 / FMT_E5M2);
    scale_a [m, k/32] and scale_b [n, k/32] are UE8M0 codes (uint8)."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    Ac, Bc = _gemm_operands(m, n, k, A, B, fmt_a, fmt_b)
    _mx_scales(m, n, k, scale_a, scale_b)
    D, code = _out(m, n, A, D, out_dtype)
    _check(load().mxfp8_gemm_ex(m, n, k, _ptr(Ac), fmt_a, _ptr(Bc), fmt_b, _ptr(scale_a), _ptr(scale_b), _ptr(D),
                                code, _stream()), "mxfp8_gemm_ex")
    return D


def mxfp8_gemm(m, n, k, A, B, scale_a, scale_b, D=None, out_dtype=None):
    """MXFP8 GEMM: scale_a [m, k/32] and scale_b [n, k/32] are UE8M0 codes (uint8)."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    Ac, Bc = _gemm_operands(m, n, k, A, B)
    _mx_scales(m, n, k, scale_a, scale_b)
    D, code = _out(m, n, A, D, out_dtype)
    _check(load().mxfp8_gemm(m, n, k, _ptr(Ac), _ptr(Bc), _ptr(scale_a), _ptr(scale_b), _ptr(D), code,
                             _stream()), "mxfp8_gemm")
    return D


def concat_mla_k(k_nope, k_rope, k=None):
    """MLA key rows: k [T, H, 192] = k_nope [T, H, 128] ++ k_rope [T, R, 64],
    R = 1 (shared by a token's heads) or H.  1-byte (float8_e4m3fn,
    float8_e5m2, uint8) or 2-byte (bfloat16, float16, int16/uint16) elements,
    copied bit for bit."""
    torch = _torch()
    if k_nope.dim() != 3 or k_nope.shape[2] != 128:
        raise ValueError("k_nope must be [T, H, 128]")
    T, H, _ = k_nope.shape
    if k_rope.dim() != 3 or k_rope.shape[0] != T or k_rope.shape[2] != 64 or k_rope.shape[1] not in (1, H):
        raise ValueError("k_rope must be [T, 1, 64] or [T, H, 64]")
    if k_rope.dtype != k_nope.dtype:
        raise TypeError("k_nope and k_rope must have the same dtype")
    esz = k_nope.element_size()
    if esz not in (1, 2):
        raise TypeError("elements must be 1 or 2 bytes, got %s" % k_nope.dtype)
    _need(k_nope, "k_nope")
    _need(k_rope, "k_rope")
    if k is None:
        k = torch.empty((T, H, 192), dtype=k_nope.dtype, device=k_nope.device)
    _need(k, "k", k_nope.dtype, (T, H, 192))
    _check(load().concat_mla_k(_ptr(k), _ptr(k_nope), _ptr(k_rope), T, H, k_rope.shape[1], esz, _stream()),
           "concat_mla_k")
    return k


def fp8g_gemm_schedule(m, n, k, mode=0, cus=None):
    """The schedule a GEMM launch takes for m x n x k on a device with `cus`
    compute units (default: the current device's): mode 0 = fp8_gemm_scaled,
    1 = mxfp8_gemm.  Host only.  Returns a dict with tile_m, tile_n, split
    (1: no K split) and split_tiles."""
    if cus is None:
        torch = _torch()
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = [ctypes.c_int(0) for _ in range(4)]
    _check(load().fp8g_gemm_schedule(int(m), int(n), int(k), int(mode), int(cus), *[ctypes.byref(o) for o in out]),
           "fp8g_gemm_schedule")
    return dict(zip(("tile_m", "tile_n", "split", "split_tiles"), (o.value for o in out)))


def fp8g_roof_mfma(blocks, iters, sink=None):
    """Queue the matrix-core roof probe on the current stream: `blocks` x 256
    threads, each wave `iters` rounds of 4 chains of the scaled 32x32x64
    instruction (blocks * 4 * iters * 4 * 131072 flops).  Returns the sink
    tensor (one float, practically never written)."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    _need(sink, "sink", torch.float32)
    _check(load().fp8g_roof_mfma(int(blocks), int(iters), _ptr(sink), _stream()), "fp8g_roof_mfma")
    return sink


def fp8g_roof_stream(src, dst, write_ratio, nontemporal_stores=0):
    """Queue the streaming roof probe on the current stream: read all of src
    (a multiple of 16 bytes), write src.nbytes / write_ratio bytes of dst
    (write_ratio 1 or 4) with write-back (0) or non-temporal (1) stores."""
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes // max(int(write_ratio), 1):
        raise ValueError("dst must hold src.nbytes / write_ratio bytes")
    _check(load().fp8g_roof_stream(_ptr(src), nbytes, _ptr(dst), int(write_ratio), int(nontemporal_stores),
                                   _stream()), "fp8g_roof_stream")
    return dst
