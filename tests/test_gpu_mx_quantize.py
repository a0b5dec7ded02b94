"""GPU parity of mxfp8_quantize: bit-exact E4M3 codes and UE8M0 scale codes
vs the oracle (oracle.quant.mx_quantize)."""

import numpy as np
import pytest

import synth
from gpu_util import alignment, say, to_dev, to_host
from oracle import quant

pytestmark = pytest.mark.gpu


def check_mx(fp8g, x, what):
    say("mx quantize", what, x.shape)
    q, s = fp8g.mxfp8_quantize(to_dev(x))
    q, s = to_host(q), to_host(s)
    qr, sr = quant.mx_quantize(x)
    if not np.array_equal(s, sr):
        r, j = np.argwhere(s != sr)[0]
        raise AssertionError("%s: %d scale codes differ; first at (%d,%d): gpu %d oracle %d (block amax %r)"
                             % (what, int((s != sr).sum()), r, j, s[r, j], sr[r, j],
                                float(np.abs(x[r, 32 * j:32 * j + 32]).max())))
    if not np.array_equal(q, qr):
        r, c = np.argwhere(q != qr)[0]
        raise AssertionError("%s: %d codes differ; first at (%d,%d): x=%r gpu=%02x oracle=%02x"
                             % (what, int((q != qr).sum()), r, c, x[r, c], q[r, c], qr[r, c]))


# flat sizes on both sides of the grid-stride step (256 threads x 4 float4 per
# lane = 4096 elements per workgroup iteration) and of the grid cap
SHAPES = [(1, 32), (3, 64), (7, 96), (5, 160), (1000, 32), (128, 4096), (33, 8192), (4097, 64), (2, 40000 // 32 * 32)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_mx_quantize_shapes(gpu_lib, rows, cols):
    w = synth.Workload("mxq", rows, rows, cols, "b", "blockpow2", "blockpow2", "mx", 13)
    check_mx(gpu_lib, synth.draw(w, "a"), "shape %dx%d" % (rows, cols))


def edge_blocks():
    """One block per row of 32: the exponent search's boundaries and the
    clamps, and casts of tiny and signed-zero elements."""
    rows = []
    rng = np.random.default_rng(7)

    def block(amax, fill):
        b = np.asarray(fill, np.float32).copy()
        b[0] = amax
        return b

    for k in range(-20, 21):
        top = np.float32(np.ldexp(448.0, k))
        fill = (rng.standard_normal(32) * float(top) / 8).astype(np.float32)
        fill = np.clip(fill, -top, top)
        rows.append(block(top, fill))                                            # amax = 448 * 2^k: e = k
        rows.append(block(np.nextafter(top, np.float32(np.inf)), fill))          # just above: e = k + 1
        rows.append(block(np.nextafter(top, np.float32(0.0)), fill))             # just below: e = k
        rows.append(block(-top, fill))                                            # amax from a negative value
    rows.append(np.zeros(32, np.float32))                                         # all zero: code 0
    z = np.zeros(32, np.float32)
    z[1::2] = -0.0
    rows.append(z)                                                                # signed zeros
    rows.append(block(np.float32(1e-40), np.full(32, 3e-45, np.float32)))         # subnormal amax: clamp to -127
    rows.append(block(np.float32(np.ldexp(448.0, -127)), np.zeros(32, np.float32)))  # e = -127 exactly
    rows.append(block(np.float32(3.0e38), (rng.standard_normal(32) * 1e37).astype(np.float32)))   # huge
    rows.append(block(np.float32(448.0), np.float32(448.0) * np.ldexp(1.0, -np.arange(32)).astype(np.float32)))
    rows.append(block(np.float32(1.0), np.float32(2.0 ** -12) * np.arange(32, dtype=np.float32)))  # E4M3 subnormals
    mid = np.float32(1.0) + np.float32(2.0 ** -4)                                 # 1.0625: a tie between E4M3 codes
    rows.append(block(np.float32(1.0), np.full(32, mid, np.float32) * np.float32(0.5)))
    x = np.stack(rows).astype(np.float32)
    return np.ascontiguousarray(np.concatenate([x, x[:, ::-1]], axis=1))          # 2 blocks per row


def test_mx_quantize_edge_blocks(gpu_lib):
    check_mx(gpu_lib, edge_blocks(), "edge blocks")


def test_mx_quantize_c5_operands(gpu_lib):
    """The 4096x14336x4096 MXFP8 workload: A (4096 x 4096) in full, the first
    2048 rows of B."""
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    check_mx(gpu_lib, synth.draw(w, "a"), "c5 A")
    check_mx(gpu_lib, synth.draw(w, "b", slice(0, 2048)), "c5 B rows 0..2047")


def test_mx_quantize_feeds_mxfp8_gemm(gpu_lib):
    """GPU quantizer -> GPU MXFP8 GEMM equals oracle quantizer -> oracle GEMM
    within the GEMM bound (the quantizer's output is exact, so this checks the
    hand-off: layouts of codes and scale bytes)."""
    from gpu_util import assert_gemm_close
    from oracle import gemm
    w = synth.Workload("mxh", 200, 136, 512, "b", "blockpow2", "blockpow2", "mx", 14)
    XA, XB = synth.draw(w, "a"), synth.draw(w, "b")
    qa, ea = gpu_lib.mxfp8_quantize(to_dev(XA))
    qb, eb = gpu_lib.mxfp8_quantize(to_dev(XB))
    D = to_host(gpu_lib.mxfp8_gemm(w.M, w.N, w.K, qa, qb, ea, eb))
    oa, oea = quant.mx_quantize(XA)
    ob, oeb = quant.mx_quantize(XB)
    assert_gemm_close(D, gemm.mxfp8_gemm(oa, ob, oea, oeb), gemm.mxfp8_gemm_weight(oa, ob, oea, oeb), "bf16",
                      "mx quantize -> gemm", alignment(oa, ob, ea=oea, eb=oeb))


def test_mx_quantize_deterministic(gpu_lib):
    w = synth.WORKLOADS["c5_mx_4096x14336x4096"]
    x = to_dev(synth.draw(w, "a", slice(0, 512)))
    q1, s1 = gpu_lib.mxfp8_quantize(x)
    q2, s2 = gpu_lib.mxfp8_quantize(x)
    assert np.array_equal(to_host(q1), to_host(q2)) and np.array_equal(to_host(s1), to_host(s2))
