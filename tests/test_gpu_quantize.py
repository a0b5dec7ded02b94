"""GPU parity of fp8_quantize_rowwise and fp8_quantize_ex (bf16 input, one
scale per tensor, E5M2 output): bit-exact codes and scales vs the oracle."""

import os

import numpy as np
import pytest

import synth
from gpu_util import alignment, oracle_quantize_rows, say, to_dev, to_host
from oracle import quant

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(fp8g, x):
    q, s = fp8g.fp8_quantize_rowwise(to_dev(x))
    return to_host(q), to_host(s)


def check_rows(fp8g, x, what):
    say("quantize", what, x.shape)
    q, s = run(fp8g, x)
    qr, sr = oracle_quantize_rows(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), what + ": scales differ"
    if not np.array_equal(q, qr):
        r, c = np.argwhere(q != qr)[0]
        raise AssertionError("%s: %d codes differ; first at (%d,%d): x=%r gpu=%02x oracle=%02x"
                             % (what, int((q != qr).sum()), r, c, x[r, c], q[r, c], qr[r, c]))


# shapes exercise every kernel variant: one wave per row (up to 1024 columns),
# one workgroup per row with the row in registers (up to 16384), the two-pass
# workgroup path (longer rows), and the element-wise path (cols % 4 != 0)
SHAPES = [(1, 4), (3, 16), (5, 60), (7, 256), (9, 260), (128, 512), (6, 1000), (4, 2048), (33, 4096),
          (130, 8192), (3, 8196), (4, 10000), (5, 257), (9, 1002), (2, 1), (3, 3), (64, 4099),
          (3, 16384), (5, 16388), (2, 40000)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_quantize_shapes(gpu_lib, rows, cols):
    w = synth.Workload("q", rows, rows, cols, "a", "rowfactor_outlier", "normal", "rowwise", 11)
    check_rows(gpu_lib, synth.draw(w, "a"), "rowfactor_outlier")


def edge_rows(cols=64):
    t = 2.0 ** -149
    rows = [
        np.zeros(cols),                                       # all zero -> s = 0, +0 codes
        np.where(np.arange(cols) % 2 == 0, 0.0, -0.0),        # signed zeros
        np.r_[t, -t, np.zeros(cols - 2)],                     # amax/448 underflows -> s = 0, signed zeros
        np.r_[1075 * t, 300 * t, -1075 * t, np.zeros(cols - 3)],   # subnormal s: saturation path
        np.r_[896.0, 1.0, -3.0, 0.5, 2.0 ** -8, 15 * 2.0 ** -9, -2.0 ** -12, np.zeros(cols - 7)],
        np.r_[-5.0, np.zeros(cols - 1)],                      # single nonzero, negative
        np.linspace(-448, 448, cols),                         # s = 1: plain cast incl. exact grid points
        np.r_[448.0, (np.arange(1, cols) + 0.5) * 2.0 ** -9],  # subnormal-range midpoints at s = 1
        np.full(cols, 3.0e38),                                # huge, all equal
        np.r_[1e-38, 3e-39, -7e-40, np.zeros(cols - 3)],      # amax is itself near/below fp32 normal min
        np.r_[2.0 ** 100, 2.0 ** 50, -1.0, np.zeros(cols - 3)],  # wide dynamic range: tiny codes flush to 0
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("cols", [64, 67])
def test_quantize_edge_rows(gpu_lib, cols):
    check_rows(gpu_lib, edge_rows(cols), "edge rows, cols=%d" % cols)


def test_quantize_empty(gpu_lib):
    import torch
    x = torch.zeros((0, 16), dtype=torch.float32, device="cuda")
    q, s = gpu_lib.fp8_quantize_rowwise(x)
    assert q.shape == (0, 16) and s.shape == (0,)
    x = torch.zeros((3, 0), dtype=torch.float32, device="cuda")
    s = torch.full((3,), 7.0, device="cuda")
    q, s = gpu_lib.fp8_quantize_rowwise(x, scale=s)
    assert to_host(s).tolist() == [0.0, 0.0, 0.0]


def _thresholds():
    vals = []
    for line in open(os.path.join(GOLDEN, "e4m3_thresholds.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            vals.append(int(line.split()[1], 16))
    assert len(vals) == 126
    return vals


def test_cast_every_fp32_pattern_up_to_448(gpu_lib):
    """Rows [448 x4, p .. p+8187] give s = 1, so q = cast(x) exactly: every
    non-negative fp32 pattern up to 448, and its negative, through the main
    (register-resident, 8192-column) kernel.  Expected codes come from the
    oracle's thresholds (tests/golden/e4m3_thresholds.txt)."""
    import torch
    thr = torch.tensor(_thresholds(), dtype=torch.int64, device="cuda")
    top = int(np.array([448.0], np.float32).view(np.uint32)[0])
    per_row = 8188
    rows = 16384
    head = torch.full((rows, 4), 448.0, dtype=torch.float32, device="cuda")
    start = 0
    while start <= top:
        n = min(rows * per_row, top + 1 - start)
        r = (n + per_row - 1) // per_row
        bits = torch.arange(start, start + r * per_row, dtype=torch.int64, device="cuda")
        bits = torch.clamp(bits, max=top)
        x = torch.cat([head[:r], bits.to(torch.int32).view(torch.float32).view(r, per_row)], dim=1).contiguous()
        want = torch.bucketize(bits, thr, right=True).to(torch.uint8).view(r, per_row)
        for sign in (1.0, -1.0):
            say("exhaustive cast", hex(start), "sign", sign)
            q, s = gpu_lib.fp8_quantize_rowwise(x * sign)
            assert bool((s == 1.0).all())
            qc = q.view(torch.uint8)
            assert bool((qc[:, :4] == (0x7E if sign > 0 else 0xFE)).all())
            exp = want if sign > 0 else (want | 0x80)
            bad = (qc[:, 4:] != exp)
            if bool(bad.any()):
                i = int(torch.nonzero(bad.view(-1))[0])
                raise AssertionError("pattern 0x%08x sign %+d: gpu %02x oracle %02x"
                                     % (int(bits[i]), int(sign), int(qc[:, 4:].reshape(-1)[i]),
                                        int(exp.reshape(-1)[i])))
        start += n


def test_quantize_division_near_rounding_boundaries(gpu_lib):
    """Quotients x / s within 3 fp32 ulps of every E4M3 rounding boundary (both
    signs), for 2048 row scales log-uniform in [2^-20, 2^20], scales whose
    significand is all ones or exactly 1, and scales below the smallest normal
    fp32.  The codes match the oracle only if the kernel's quotient is the
    correctly rounded fp32 division x / s for every one of them."""
    thr = np.array(_thresholds(), dtype=np.uint32).view(np.float32).astype(np.float64)   # 126 boundaries
    u = synth.uniform(synth.stream_key(0x5EED, 1), 0, 2048)
    s0 = np.concatenate([np.exp2(40.0 * u - 20.0),
                         np.ldexp(2.0 - 2.0 ** -23, np.arange(-20, 20)),       # significand all ones
                         np.ldexp(1.0, np.arange(-20, 20)),                    # powers of two
                         np.ldexp(1.0 + u[:16], -130)])                        # subnormal scales
    amax = (448.0 * s0).astype(np.float32)
    s = amax / np.float32(448.0)                                               # the scale each row gets
    cols = 1792
    x = np.zeros((len(s0), cols), np.float32)
    x[:, 0] = amax
    base = (thr[None, :] * s.astype(np.float64)[:, None]).astype(np.float32)   # RN(m s)
    c = 1
    for k in range(-3, 4):
        v = base.copy()
        for _ in range(abs(k)):
            v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(0.0))
        for sign in (1.0, -1.0):
            x[:, c:c + thr.size] = np.float32(sign) * v
            c += thr.size
    assert c <= cols
    check_rows(gpu_lib, x, "division near rounding boundaries")


@pytest.mark.parametrize("side,rows", [("a", None), ("b", slice(0, 4096))])
def test_quantize_ffn_up_operands(gpu_lib, side, rows):
    """The 8192x22016x8192 FFN-up workload: activations (8192 x 8192, per-row
    log-uniform factors and x50 outliers) in full; weights (N(0, 0.02)) on the
    first 4096 channels."""
    w = synth.WORKLOADS["c4_ffn_up_8192x22016x8192"]
    check_rows(gpu_lib, synth.draw(w, side, rows), "ffn_up side " + side)


def test_quantize_deterministic(gpu_lib):
    w = synth.WORKLOADS["c3_8192x2048x8192"]
    x = to_dev(synth.draw(w, "a", slice(0, 512)))
    q1, s1 = gpu_lib.fp8_quantize_rowwise(x)
    q2, s2 = gpu_lib.fp8_quantize_rowwise(x)
    import torch
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s1, s2)


# ---- fp8_quantize_ex: bf16 input, and one scale per tensor

def _bf16_bits(x32):
    """fp32 -> bf16 bit patterns (round to nearest even), via torch on the CPU."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


BF16_SHAPES = [(1, 8), (3, 16), (7, 512), (5, 520), (130, 2048), (9, 4096), (4, 8192), (3, 16384), (2, 32776),
               (6, 1000), (5, 257), (2, 3)]


@pytest.mark.parametrize("rows,cols", BF16_SHAPES)
def test_quantize_bf16_rows(gpu_lib, rows, cols):
    """bf16 rows through every kernel variant (8 elements per 16-byte load, the
    two-pass path, the element-wise path): codes and scales equal the oracle's
    row-wise quantizer on the exactly converted fp32 tensor."""
    w = synth.Workload("qb", rows, rows, cols, "a", "rowfactor_outlier", "normal", "rowwise", 23)
    bits = _bf16_bits(synth.draw(w, "a"))
    say("quantize bf16 rows", rows, cols)
    q, s = gpu_lib.fp8_quantize_ex(_dev_bf16(bits))
    qr, sr = quant.quantize_rowwise(quant.bf16_to_f32(bits))
    assert np.array_equal(to_host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(to_host(q), qr)


def test_quantize_bf16_edge_rows(gpu_lib):
    bits = _bf16_bits(edge_rows(64))
    q, s = gpu_lib.fp8_quantize_ex(_dev_bf16(bits))
    qr, sr = quant.quantize_rowwise(quant.bf16_to_f32(bits))
    assert np.array_equal(to_host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(to_host(q), qr)


def _tensor_cases():
    rng_key = synth.stream_key(0x7E50, 1)
    out = []
    for (r, c) in [(1, 1), (3, 5), (1, 7), (33, 1001), (1000, 1001), (4096, 4096), (2, 3)]:
        x = synth.normal(rng_key, 0, r * c).astype(np.float32).reshape(r, c)
        out.append(("normal %dx%d" % (r, c), x))
    x = synth.normal(rng_key, 0, 999 * 17).astype(np.float32).reshape(999, 17)
    x[-1, -1] = 1.0e6                                   # amax in the scalar tail (past the last whole vector)
    out.append(("amax in tail", x))
    x = synth.normal(rng_key, 0, 512 * 2048).astype(np.float32).reshape(512, 2048)
    x[300, 1000] = -3.0e5                               # amax in the middle, negative
    out.append(("amax in middle", x))
    out.append(("all zero", np.zeros((64, 64), np.float32)))
    return out


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_quantize_per_tensor(gpu_lib, in_dtype):
    """One scale for the tensor: the amax of every element across all
    workgroups (atomic max) and the cast with it, bit-exact vs the oracle."""
    for name, x in _tensor_cases():
        say("quantize per tensor", in_dtype, name, x.shape)
        if in_dtype == "bf16":
            bits = _bf16_bits(x)
            xin, x32 = _dev_bf16(bits), quant.bf16_to_f32(bits)
        else:
            xin, x32 = to_dev(x), x
        q, s = gpu_lib.fp8_quantize_ex(xin, per_tensor=True)
        qr, sr = quant.quantize_tensorwise(x32)
        assert np.array_equal(to_host(s).view(np.uint32), sr.view(np.uint32)), (name, to_host(s), sr)
        qg = to_host(q)
        if not np.array_equal(qg, qr):
            i = np.argwhere(qg != qr)[0]
            raise AssertionError("%s: %d codes differ, first at %s" % (name, int((qg != qr).sum()), tuple(i)))


def test_quantize_ex_fp32_rows_equal_rowwise(gpu_lib):
    """fp8_quantize_ex on fp32 rows is fp8_quantize_rowwise."""
    w = synth.WORKLOADS["c3_8192x2048x8192"]
    x = to_dev(synth.draw(w, "b", slice(0, 512)))
    q1, s1 = gpu_lib.fp8_quantize_rowwise(x)
    q2, s2 = gpu_lib.fp8_quantize_ex(x)
    assert np.array_equal(to_host(q1), to_host(q2)) and np.array_equal(to_host(s1), to_host(s2))


# ---- E5M2 output (fp8_quantize_ex with fmt = E5M2): scale amax / 57344

E5M2 = 1


def check_ex(fp8g, x, what, per_tensor=False, bf16=False):
    """fp8_quantize_ex to E5M2 vs the oracle on the same (bf16-converted) values."""
    say("quantize e5m2", what, x.shape, "per tensor" if per_tensor else "per row", "bf16" if bf16 else "f32")
    if bf16:
        bits = _bf16_bits(x)
        xin, x32 = _dev_bf16(bits), quant.bf16_to_f32(bits)
    else:
        xin, x32 = to_dev(x), x
    q, s = fp8g.fp8_quantize_ex(xin, per_tensor=per_tensor, fmt=E5M2)
    import torch
    assert q.dtype == torch.float8_e5m2
    qg, sg = q.view(torch.uint8).cpu().numpy(), to_host(s)
    if per_tensor:
        qr, sr = quant.quantize_tensorwise(x32, "e5m2")
    else:
        qr, sr = quant.quantize_rowwise(x32, "e5m2")
    assert np.array_equal(sg.view(np.uint32), sr.view(np.uint32)), what + ": scales differ"
    if not np.array_equal(qg, qr):
        r, c = np.argwhere(qg != qr)[0]
        raise AssertionError("%s: %d codes differ; first at (%d,%d): x=%r gpu=%02x oracle=%02x"
                             % (what, int((qg != qr).sum()), r, c, x32[r, c], qg[r, c], qr[r, c]))


E5M2_SHAPES = [(1, 4), (5, 60), (9, 260), (128, 512), (6, 1000), (33, 4096), (130, 8192), (4, 10000),
               (5, 257), (3, 3), (3, 16384), (2, 40000)]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rows,cols", E5M2_SHAPES)
def test_quantize_e5m2_rows(gpu_lib, rows, cols, bf16):
    w = synth.Workload("q5", rows, rows, cols, "a", "rowfactor_outlier", "normal", "rowwise", 29)
    check_ex(gpu_lib, synth.draw(w, "a"), "rowfactor_outlier", bf16=bf16)


def e5m2_edge_rows(cols=64):
    t = 2.0 ** -149
    rows = [
        np.zeros(cols),
        np.where(np.arange(cols) % 2 == 0, 0.0, -0.0),
        np.r_[t, -t, np.zeros(cols - 2)],                            # amax/57344 underflows: s = 0
        np.r_[2 ** 20 * t, 300 * t, -(2 ** 20) * t, np.zeros(cols - 3)],   # subnormal s
        np.r_[114688.0, 1.0, -3.0, 0.5, 2.0 ** -15, 3 * 2.0 ** -16, -2.0 ** -20, np.zeros(cols - 7)],
        np.linspace(-57344, 57344, cols),                            # s = 1: plain cast
        np.r_[57344.0, (np.arange(1, cols) + 0.5) * 2.0 ** -16],     # subnormal midpoints at s = 1
        np.full(cols, 3.0e38),
        np.r_[2.0 ** 100, 2.0 ** 70, -1.0, np.zeros(cols - 3)],
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("cols", [64, 67])
def test_quantize_e5m2_edge_rows(gpu_lib, cols):
    check_ex(gpu_lib, e5m2_edge_rows(cols), "e5m2 edge rows, cols=%d" % cols)
    check_ex(gpu_lib, edge_rows(cols), "e4m3 edge rows as e5m2, cols=%d" % cols)


@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_e5m2_per_tensor(gpu_lib, bf16):
    for name, x in _tensor_cases():
        check_ex(gpu_lib, x, name, per_tensor=True, bf16=bf16)


def test_quantize_e5m2_division_near_rounding_boundaries(gpu_lib):
    """Quotients within 3 fp32 ulps of every E5M2 rounding boundary (the
    midpoints between adjacent magnitudes), both signs, over 2048 log-uniform
    row scales and scales with all-ones or unit significands."""
    from oracle import e5m2
    mags = e5m2.DECODE_TABLE[:0x7C]
    thr = (mags[:-1] + mags[1:]) / 2                                    # 123 boundaries, exact in fp32
    u = synth.uniform(synth.stream_key(0x5EED, 2), 0, 2048)
    s0 = np.concatenate([np.exp2(40.0 * u - 20.0), np.ldexp(2.0 - 2.0 ** -23, np.arange(-20, 20)),
                         np.ldexp(1.0, np.arange(-20, 20))])
    amax = (57344.0 * s0).astype(np.float32)
    s = amax / np.float32(57344.0)
    cols = 7 * 2 * thr.size + 1
    x = np.zeros((len(s0), cols), np.float32)
    x[:, 0] = amax
    base = (thr[None, :] * s.astype(np.float64)[:, None]).astype(np.float32)
    c = 1
    for k in range(-3, 4):
        v = base.copy()
        for _ in range(abs(k)):
            v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(0.0))
        for sign in (1.0, -1.0):
            x[:, c:c + thr.size] = np.float32(sign) * v
            c += thr.size
    check_ex(gpu_lib, x, "e5m2 division near rounding boundaries")


def test_quantize_e5m2_feeds_e5m2_gemm(gpu_lib):
    """GPU E5M2 quantizer -> GPU GEMM with E5M2 activations and E4M3 weights ==
    oracle quantizers -> oracle GEMM within the GEMM bound."""
    from gpu_util import assert_gemm_close
    from oracle import gemm
    w = synth.Workload("q5g", 300, 260, 1024, "a", "rowfactor_outlier", "normal", "rowwise", 31)
    XA, XB = synth.draw(w, "a"), synth.draw(w, "b")
    qa, sa = gpu_lib.fp8_quantize_ex(to_dev(XA), fmt=E5M2)
    qb, sb = gpu_lib.fp8_quantize_rowwise(to_dev(XB))
    D = to_host(gpu_lib.fp8_gemm_scaled_ex(w.M, w.N, w.K, qa, E5M2, qb, 0, sa, sb))
    oa, osa = quant.quantize_rowwise(XA, "e5m2")
    ob, osb = quant.quantize_rowwise(XB)
    assert_gemm_close(D, gemm.gemm_scaled(oa, ob, osa, osb, "e5m2", "e4m3"),
                      gemm.gemm_scaled_weight(oa, ob, osa, osb, "e5m2", "e4m3"), "bf16", "e5m2 quantize -> gemm",
                      alignment(oa, ob, osa, osb, fmt_a="e5m2", fmt_b="e4m3"))


# The quantize benchmark's six modes (fp8_quantize_ex on the 8192 x 8192 FFN-up
# activations: fp32 or bf16 input, one scale per row or per tensor, E4M3 or
# E5M2 codes), at that full size, against the plain C++ oracle bit for bit.  A
# per-tensor scale is the row-wise rule applied to the tensor as one row.
BENCH_MODES = [("f32_row_e4m3", False, False, "e4m3"), ("bf16_row_e4m3", True, False, "e4m3"),
               ("f32_tensor_e4m3", False, True, "e4m3"), ("bf16_tensor_e4m3", True, True, "e4m3"),
               ("f32_row_e5m2", False, False, "e5m2"), ("bf16_row_e5m2", True, False, "e5m2")]


@pytest.fixture(scope="module")
def ffn_up_activations():
    return synth.draw(synth.WORKLOADS["c4_ffn_up_8192x22016x8192"], "a")


@pytest.mark.parametrize("name,bf16,per_tensor,fmt", BENCH_MODES, ids=[m[0] for m in BENCH_MODES])
def test_quantize_bench_modes_full_size(gpu_lib, ffn_up_activations, name, bf16, per_tensor, fmt):
    import torch
    from oracle import cpp_oracle
    x = ffn_up_activations
    if bf16:
        bits = _bf16_bits(x)
        xin, x32 = _dev_bf16(bits), quant.bf16_to_f32(bits)
    else:
        xin, x32 = to_dev(x), x
    say("quantize bench mode", name, x.shape)
    q, s = gpu_lib.fp8_quantize_ex(xin, per_tensor=per_tensor, fmt=E5M2 if fmt == "e5m2" else 0)
    torch.cuda.synchronize()
    qg, sg = q.view(torch.uint8).cpu().numpy(), to_host(s)
    del q, xin
    if per_tensor:
        qr, sr = cpp_oracle.quantize_rowwise(x32.reshape(1, -1), fmt)
        qr = qr.reshape(x.shape)
    else:
        qr, sr = cpp_oracle.quantize_rowwise(x32, fmt)
    assert np.array_equal(sg.view(np.uint32), sr.view(np.uint32)), name + ": scales differ"
    if not np.array_equal(qg, qr):
        r, c = np.argwhere(qg != qr)[0]
        raise AssertionError("%s: %d codes differ; first at (%d,%d): x=%r gpu=%02x oracle=%02x"
                             % (name, int((qg != qr).sum()), r, c, x32[r, c], qg[r, c], qr[r, c]))
