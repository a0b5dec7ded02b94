"""The C ABI on the CPU: the library loads, exports every declared function,
and rejects bad arguments with the documented status before any HIP call.

Pointers here are plain integers that are never dereferenced.  A call that
passes every host-side check goes on to queue its kernel; without a device
that returns ERR_HIP.  Such calls are made only where no device is visible
(passes_checks), so that no kernel is ever launched on these addresses.
"""

import ctypes

import pytest

import fp8_scaled_gemm_amd as fp8g

OK, NULL, SHAPE, ALIGN, DTYPE, OVERLAP, UNSUPPORTED, HIP = range(8)
P = 0x100000          # a fake, 16-byte aligned "device" address
S = 0                 # null stream


def P_(off):
    return ctypes.c_void_p(P + off)


def _device_visible():
    # counting devices does not initialise the GPU on this image
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return True          # unknown: treat as visible, launch nothing


DEVICE_VISIBLE = _device_visible()


def passes_checks(call):
    """A call that passes every host-side check would queue its kernel: made
    only where no device is visible (it then returns ERR_HIP, or OK where the
    runtime queues lazily), never on these addresses on a GPU."""
    if DEVICE_VISIBLE:
        return
    assert call() in (OK, HIP)


@pytest.fixture(scope="module")
def lib():
    return fp8g.load()


def test_exports_every_header_function(lib):
    names = fp8g.header_functions()
    assert set(names) == {"fp8_quantize_rowwise", "fp8_quantize_ex", "mxfp8_quantize", "fp8_gemm_scaled",
                          "fp8_gemm_scaled_noalloc", "mxfp8_gemm", "fp8_gemm_scaled_ex", "mxfp8_gemm_ex", "concat_mla_k",
                          "fp8g_gemm_schedule", "fp8g_roof_mfma", "fp8g_roof_stream", "fp8g_status_string"}
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(8):
        assert fp8g.status_string(st)
    assert fp8g.status_string(99) == "unknown status"


def gemm(lib, fn, m, n, k, A=P_(0), B=P_(1 << 30), sa=P_(2 << 30), sb=P_(3 << 30), D=P_(4 << 30), out=0,
         fa=1, fb=0):
    if fn.endswith("_ex"):      # the format-per-operand variants: E5M2 A, E4M3 B unless given
        return getattr(lib, fn)(m, n, k, A, fa, B, fb, sa, sb, D, out, ctypes.c_void_p(S))
    return getattr(lib, fn)(m, n, k, A, B, sa, sb, D, out, ctypes.c_void_p(S))


@pytest.mark.parametrize("fn", ["fp8_gemm_scaled", "fp8_gemm_scaled_noalloc", "mxfp8_gemm", "fp8_gemm_scaled_ex",
                                "mxfp8_gemm_ex"])
def test_gemm_argument_checks(lib, fn):
    assert gemm(lib, fn, -1, 4, 64) == SHAPE
    assert gemm(lib, fn, 4, -1, 64) == SHAPE
    assert gemm(lib, fn, 4, 4, -32) == SHAPE
    assert gemm(lib, fn, 4, 4, 64, out=2) == DTYPE
    assert gemm(lib, fn, 4, 4, 64, out=-1) == DTYPE
    assert gemm(lib, fn, 0, 4, 64) == OK           # empty output: no-op
    assert gemm(lib, fn, 4, 0, 64) == OK
    assert gemm(lib, fn, 0, 0, 0, A=None, B=None, sa=None, sb=None, D=None) == OK
    assert gemm(lib, fn, 4, 4, 64, D=None) == NULL
    assert gemm(lib, fn, 4, 4, 64, A=None) == NULL
    assert gemm(lib, fn, 4, 4, 64, B=None) == NULL
    assert gemm(lib, fn, 4, 4, 64, sa=None) == NULL
    assert gemm(lib, fn, 4, 4, 64, sb=None) == NULL
    assert gemm(lib, fn, 4, 4, 64, A=P_(8)) == ALIGN
    assert gemm(lib, fn, 4, 4, 64, B=P_((1 << 30) + 4)) == ALIGN
    assert gemm(lib, fn, 4, 4, 64, D=P_((4 << 30) + 2)) == ALIGN
    assert gemm(lib, fn, 4, 4, 64, sa=P_((2 << 30) + 1)) == ALIGN
    # D overlaps A / B / a scale array
    assert gemm(lib, fn, 4, 4, 64, D=P_(0)) == OVERLAP
    assert gemm(lib, fn, 4, 4, 64, D=P_((1 << 30) + 16)) == OVERLAP
    assert gemm(lib, fn, 4, 4, 64, D=P_((3 << 30) - 16)) == OVERLAP
    # adjacent but not overlapping is fine up to the launch, which fails without a GPU
    passes_checks(lambda: gemm(lib, fn, 4, 4, 64, D=P_(4 * 64)))


@pytest.mark.parametrize("fn", ["fp8_gemm_scaled_ex", "mxfp8_gemm_ex"])
def test_gemm_format_checks(lib, fn):
    for fa, fb in ((0, 0), (0, 1), (1, 0), (1, 1)):
        assert gemm(lib, fn, 4, 4, 64, fa=fa, fb=fb, D=None) == NULL     # formats accepted, checks go on
    for fa, fb in ((2, 0), (0, 2), (-1, 0), (0, 4)):
        assert gemm(lib, fn, 4, 4, 64, fa=fa, fb=fb) == DTYPE
        assert gemm(lib, fn, 0, 4, 64, fa=fa, fb=fb) == DTYPE            # checked before the empty no-op
    assert gemm(lib, fn, -1, 4, 64, fa=2) == SHAPE


def test_mx_k_must_be_multiple_of_32(lib):
    for k in (16, 48, 33, 1):
        assert gemm(lib, "mxfp8_gemm", 4, 4, k) == SHAPE
        assert gemm(lib, "mxfp8_gemm_ex", 4, 4, k) == SHAPE


def test_scaled_k_must_be_multiple_of_16(lib):
    for k in (8, 24, 33, 1):
        assert gemm(lib, "fp8_gemm_scaled", 4, 4, k) == UNSUPPORTED
        assert gemm(lib, "fp8_gemm_scaled_noalloc", 4, 4, k) == UNSUPPORTED
        assert gemm(lib, "fp8_gemm_scaled_ex", 4, 4, k) == UNSUPPORTED


def test_k_zero_needs_no_operands(lib):
    # the empty sum: A and B may be NULL; the call proceeds to the launch
    passes_checks(lambda: gemm(lib, "fp8_gemm_scaled", 4, 4, 0, A=None, B=None))


def test_huge_sizes_rejected(lib):
    assert gemm(lib, "fp8_gemm_scaled", 1 << 40, 1 << 40, 1 << 20) == UNSUPPORTED


@pytest.mark.parametrize("fn", ["fp8_gemm_scaled", "fp8_gemm_scaled_noalloc", "mxfp8_gemm", "fp8_gemm_scaled_ex",
                                "mxfp8_gemm_ex"])
def test_gemm_32bit_panel_limits(lib, fn):
    """k < 2^23, m < 2^31, and a 256-row panel of D below 2^31 bytes: n < 2^22
    for bf16 output, n < 2^21 for fp32 output.  Just inside each limit the call
    passes the host checks (and fails only at the launch, without a GPU)."""
    far = 1 << 44                                   # operands far apart: no overlap at these sizes
    kw = dict(B=P_(far), sa=P_(2 * far), sb=P_(3 * far), D=P_(4 * far))
    assert gemm(lib, fn, 4, 4, 1 << 23, **kw) == UNSUPPORTED
    passes_checks(lambda: gemm(lib, fn, 4, 4, (1 << 23) - 128, **kw))
    assert gemm(lib, fn, 1 << 31, 4, 128, **kw) == UNSUPPORTED
    assert gemm(lib, fn, 4, (1 << 22) + 1, 128, out=0, **kw) == UNSUPPORTED
    passes_checks(lambda: gemm(lib, fn, 4, 1 << 22, 128, out=0, **kw))
    assert gemm(lib, fn, 4, (1 << 21) + 1, 128, out=1, **kw) == UNSUPPORTED
    passes_checks(lambda: gemm(lib, fn, 4, 1 << 21, 128, out=1, **kw))
    # n so large that n * 256 * element size would overflow 64 bits: still rejected
    assert gemm(lib, fn, 1, 1 << 55, 32, **kw) == UNSUPPORTED


def test_quantize_rows_limit(lib):
    far = 1 << 44
    assert lib.fp8_quantize_rowwise(P_(0), 1 << 31, 1, P_(far), P_(2 * far), ctypes.c_void_p(S)) == UNSUPPORTED
    assert lib.fp8_quantize_ex(P_(0), 0, 1 << 31, 1, 0, 0, P_(far), P_(2 * far), ctypes.c_void_p(S)) == UNSUPPORTED
    # per tensor has no per-row grid: the same extent passes the host checks
    passes_checks(lambda: lib.fp8_quantize_ex(P_(0), 0, 1 << 31, 1, 1, 0, P_(far), P_(2 * far), ctypes.c_void_p(S)))


def quant(lib, x=P_(0), rows=8, cols=64, q=P_(1 << 30), s=P_(2 << 30)):
    return lib.fp8_quantize_rowwise(x, rows, cols, q, s, ctypes.c_void_p(S))


def test_quantize_argument_checks(lib):
    assert quant(lib, rows=-1) == SHAPE
    assert quant(lib, cols=-1) == SHAPE
    assert quant(lib, rows=0, x=None, q=None, s=None) == OK
    assert quant(lib, s=None) == NULL
    assert quant(lib, x=None) == NULL
    assert quant(lib, q=None) == NULL
    assert quant(lib, x=P_(4)) == ALIGN
    assert quant(lib, q=P_((1 << 30) + 1)) == ALIGN
    assert quant(lib, s=P_((2 << 30) + 8)) == ALIGN
    assert quant(lib, q=P_(64)) == OVERLAP                    # q inside x
    assert quant(lib, s=P_((1 << 30) + 16)) == OVERLAP        # scale inside q
    passes_checks(lambda: quant(lib, cols=0, x=None, q=None))    # empty rows: only scales written


def qex(lib, x=P_(0), dt=0, rows=8, cols=64, g=0, q=P_(1 << 30), s=P_(2 << 30), fmt=1):
    return lib.fp8_quantize_ex(x, dt, rows, cols, g, fmt, q, s, ctypes.c_void_p(S))


def test_quantize_ex_argument_checks(lib):
    for g in (0, 1):
        assert qex(lib, rows=-1, g=g) == SHAPE
        assert qex(lib, cols=-1, g=g) == SHAPE
        assert qex(lib, s=None, g=g) == NULL
        assert qex(lib, x=None, g=g) == NULL
        assert qex(lib, q=None, g=g) == NULL
        assert qex(lib, x=P_(8), g=g) == ALIGN
        assert qex(lib, s=P_((2 << 30) + 4), g=g) == ALIGN
        assert qex(lib, q=P_(256), g=g) == OVERLAP                       # q inside x (fp32: 2 KB)
    assert qex(lib, dt=2) == DTYPE
    assert qex(lib, dt=-1) == DTYPE
    assert qex(lib, g=2) == DTYPE
    assert qex(lib, fmt=2) == DTYPE
    assert qex(lib, fmt=-1) == DTYPE
    assert qex(lib, fmt=0, s=None) == NULL and qex(lib, fmt=1, s=None) == NULL   # both formats accepted
    assert qex(lib, rows=0, x=None, q=None, s=None) == OK                # per row, empty: no-op
    assert qex(lib, rows=0, x=None, q=None, s=None, g=1) == NULL         # per tensor: the scale is written
    passes_checks(lambda: qex(lib, rows=0, x=None, q=None, g=1))
    passes_checks(lambda: qex(lib, dt=1, q=P_(1024)))                       # bf16: x is 1 KB, q adjacent
    assert qex(lib, dt=1, q=P_(1008)) == OVERLAP
    assert qex(lib, g=1, s=P_((1 << 30) + 496)) == OVERLAP               # scale [1] inside q
    assert qex(lib, rows=1 << 40, cols=1 << 30) == UNSUPPORTED


def mxq(lib, x=P_(0), rows=8, cols=64, q=P_(1 << 30), s=P_(2 << 30)):
    return lib.mxfp8_quantize(x, rows, cols, q, s, ctypes.c_void_p(S))


def test_mx_quantize_argument_checks(lib):
    assert mxq(lib, rows=-1) == SHAPE
    assert mxq(lib, cols=-32) == SHAPE
    for cols in (16, 33, 48, 1):                              # blocks of 32 along a row
        assert mxq(lib, cols=cols) == SHAPE
    assert mxq(lib, rows=0, x=None, q=None, s=None) == OK      # empty: no-op
    assert mxq(lib, cols=0, x=None, q=None, s=None) == OK
    assert mxq(lib, x=None) == NULL
    assert mxq(lib, q=None) == NULL
    assert mxq(lib, s=None) == NULL
    assert mxq(lib, x=P_(4)) == ALIGN
    assert mxq(lib, q=P_((1 << 30) + 8)) == ALIGN
    assert mxq(lib, s=P_((2 << 30) + 1)) == ALIGN
    assert mxq(lib, q=P_(1024)) == OVERLAP                     # q inside x (8 x 64 fp32 = 2 KB)
    assert mxq(lib, s=P_((1 << 30) + 256)) == OVERLAP          # scales inside q (512 B)
    passes_checks(lambda: mxq(lib, s=P_((1 << 30) + 512)))        # adjacent: proceeds to the launch
    assert mxq(lib, rows=1 << 40, cols=1 << 30) == UNSUPPORTED


def cmk(lib, k=P_(2 << 30), nope=P_(0), rope=P_(1 << 30), T=4, H=8, R=1, e=1):
    return lib.concat_mla_k(k, nope, rope, T, H, R, e, ctypes.c_void_p(S))


def test_concat_mla_k_argument_checks(lib):
    assert cmk(lib, T=-1) == SHAPE
    assert cmk(lib, H=-1) == SHAPE
    assert cmk(lib, e=3) == DTYPE
    assert cmk(lib, e=4) == DTYPE
    assert cmk(lib, T=0, k=None, nope=None, rope=None) == OK      # empty: no-op
    assert cmk(lib, H=0, k=None, nope=None, rope=None) == OK
    assert cmk(lib, R=2) == SHAPE                                   # rope heads: 1 or H
    passes_checks(lambda: cmk(lib, R=8))
    assert cmk(lib, k=None) == NULL
    assert cmk(lib, nope=None) == NULL
    assert cmk(lib, rope=None) == NULL
    assert cmk(lib, k=P_((2 << 30) + 8)) == ALIGN
    assert cmk(lib, rope=P_((1 << 30) + 2)) == ALIGN
    assert cmk(lib, k=P_(4 * 8 * 128 - 16)) == OVERLAP               # k starts inside k_nope
    passes_checks(lambda: cmk(lib, k=P_(4 * 8 * 128)))                  # adjacent
    assert cmk(lib, k=P_((1 << 30) - 16)) == OVERLAP                 # k runs into k_rope
    assert cmk(lib, T=1 << 40, H=1 << 20) == UNSUPPORTED


def test_roof_probe_argument_checks(lib):
    st = ctypes.c_void_p(S)
    assert lib.fp8g_roof_mfma(0, 10, P_(0), st) == SHAPE
    assert lib.fp8g_roof_mfma(10, 0, P_(0), st) == SHAPE
    assert lib.fp8g_roof_mfma(1 << 31, 10, P_(0), st) == SHAPE
    assert lib.fp8g_roof_mfma(10, 10, None, st) == NULL
    assert lib.fp8g_roof_stream(P_(0), -16, P_(1 << 30), 1, 0, st) == SHAPE
    assert lib.fp8g_roof_stream(P_(0), 24, P_(1 << 30), 1, 0, st) == SHAPE      # not a multiple of 16
    assert lib.fp8g_roof_stream(P_(0), 64, P_(1 << 30), 2, 0, st) == SHAPE      # ratio 1 or 4
    assert lib.fp8g_roof_stream(None, 0, None, 4, 0, st) == OK                  # empty: no-op
    assert lib.fp8g_roof_stream(None, 64, P_(1 << 30), 4, 0, st) == NULL
    assert lib.fp8g_roof_stream(P_(8), 64, P_(1 << 30), 4, 0, st) == ALIGN
    assert lib.fp8g_roof_stream(P_(0), 64, P_(48), 1, 0, st) == OVERLAP         # dst inside src
    assert lib.fp8g_roof_stream(P_(0), 64, P_(48), 4, 0, st) == OVERLAP         # 16 bytes written at 48..63
    passes_checks(lambda: lib.fp8g_roof_stream(P_(0), 64, P_(64), 1, 0, st))       # adjacent
    assert lib.fp8g_roof_stream(P_(0), 64, P_(64), 1, 2, st) == DTYPE         # store policy 0 or 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fp8g, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fp8g, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fp8g.load()


# The schedule a launch takes on a 256-CU MI355X (the host logic the launch
# itself uses; fp8g_gemm_schedule calls no HIP function).  (m, n, k, mode):
# (tile_m, tile_n, split, split_tiles).
SCHEDULES_256 = [
    ((128, 256, 512, 0), (64, 128, 1, 0)),          # C1: 2 tiles of 128: 64x128 tiles
    ((2048, 1024, 4096, 0), (64, 128, 1, 0)),       # C2: 128 tiles of 128 fill half the CUs
    ((8192, 2048, 8192, 0), (256, 256, 1, 0)),      # C3: one round of 256x256 tiles
    ((8192, 22016, 8192, 0), (256, 256, 1, 0)),     # C4
    ((4096, 14336, 4096, 1), (256, 256, 1, 0)),     # C5, MXFP8
    ((2048, 1024, 4096, 1), (128, 128, 1, 0)),      # mode (b): no 64x128 tiles, no split
    ((2048, 2048, 4096, 0), (128, 128, 1, 0)),      # 256 tiles of 128: a full round, nothing to split
    ((128, 128, 4096, 0), (128, 128, 4, 1)),        # one tile, 32 stages: split 4
    ((512, 512, 8192, 0), (128, 128, 4, 16)),
    ((1024, 1024, 8192, 0), (128, 128, 4, 64)),     # long K: the split beats 64x128 tiles
    ((1024, 1024, 4096, 0), (64, 128, 1, 0)),       # K = 4096: 64x128 tiles beat the split
    ((2048, 1024, 8192, 0), (64, 128, 1, 0)),
    ((1024, 512, 4096, 0), (64, 128, 1, 0)),
    ((512, 1024, 8192, 0), (128, 128, 4, 32)),
    ((2048, 512, 8192, 0), (128, 128, 4, 64)),
    ((1000, 1001, 8192, 0), (128, 128, 4, 64)),
    ((1000, 1024, 8192, 0), (128, 128, 4, 64)),
    ((4352, 4096, 8192, 0), (128, 128, 4, 64)),     # 272 tiles of 256 spill: 1088 of 128, last 64 split
    ((4352, 4096, 272, 0), (128, 128, 1, 0)),       # the same with a K tail: no split
    ((4352, 4096, 640, 1), (256, 128, 1, 0)),       # mode (b): 272 tiles of 256x256 (2 rounds), 544 of 256x128 (3)
    ((2600, 2900, 1024, 1), (256, 128, 1, 0)),      # 132 of 256x256, 253 of 256x128: one round either way
    ((2561, 3000, 1056, 1), (256, 256, 1, 0)),      # 264 of 256x128: twice the rounds
    ((3072, 4096, 1024, 1), (256, 256, 1, 0)),      # 192 of 256x256 (1 round) against 384 (2)
    ((4096, 8192, 2048, 1), (256, 256, 1, 0)),      # 2 rounds against 4
    ((2600, 2900, 1024, 0), (256, 128, 1, 0)),      # mode (a) the same
    ((4864, 4096, 4096, 0), (256, 128, 1, 0)),      # 304 of 256x256 (2 rounds), 608 of 256x128 (3)
    ((4000, 6400, 256, 0), (256, 256, 1, 0)),       # 400 (2 rounds) against 800 (4)
    ((3072, 4096, 1024, 0), (256, 256, 1, 0)),
    ((4352, 4096, 1024, 0), (128, 128, 1, 0)),      # the spill rule comes first
    ((1000, 1001, 272, 0), (64, 128, 1, 0)),        # K tail
    ((300, 512, 0, 0), (64, 128, 1, 0)),            # k = 0
]


@pytest.mark.parametrize("args,want", SCHEDULES_256, ids=["%dx%dx%d/%d" % a for a, _ in SCHEDULES_256])
def test_gemm_schedule(args, want):
    got = fp8g.fp8g_gemm_schedule(*args[:3], mode=args[3], cus=256)
    assert (got["tile_m"], got["tile_n"], got["split"], got["split_tiles"]) == want


def test_gemm_schedule_follows_the_cu_count():
    # 2048 x 1024 has 128 tiles of 128: on 128 CUs that is a full round
    got = fp8g.fp8g_gemm_schedule(2048, 1024, 4096, cus=128)
    assert (got["tile_m"], got["tile_n"], got["split"]) == (128, 128, 1)
    # and 32 tiles of 256 on 64 CUs: half of them, so 128x128 tiles, 128 of them, two rounds
    got = fp8g.fp8g_gemm_schedule(2048, 1024, 4096, cus=64)
    assert (got["tile_m"], got["tile_n"]) == (128, 128)
    got = fp8g.fp8g_gemm_schedule(2048, 1024, 4096, cus=1024)
    assert (got["tile_m"], got["tile_n"]) == (64, 128)


def test_gemm_schedule_argument_checks(lib):
    i = [ctypes.c_int(0) for _ in range(4)]
    r = [ctypes.byref(x) for x in i]
    assert lib.fp8g_gemm_schedule(-1, 4, 64, 0, 256, *r) == SHAPE
    assert lib.fp8g_gemm_schedule(4, 4, 64, 0, 0, *r) == SHAPE
    assert lib.fp8g_gemm_schedule(4, 4, 64, 2, 256, *r) == DTYPE
    assert lib.fp8g_gemm_schedule(4, 4, 64, 0, 256, None, r[1], r[2], r[3]) == NULL
    assert lib.fp8g_gemm_schedule(4, 4, 64, 0, 256, r[0], r[1], r[2], None) == NULL
    assert lib.fp8g_gemm_schedule(1 << 31, 4, 64, 0, 256, *r) == UNSUPPORTED
    assert lib.fp8g_gemm_schedule(4, 4, 1 << 23, 0, 256, *r) == UNSUPPORTED
    assert lib.fp8g_gemm_schedule(4, 4, 64, 1, 256, *r) == OK
    assert (i[0].value, i[1].value, i[2].value, i[3].value) == (128, 128, 1, 0)
