"""The hot path under HIP graph capture: quantize both operands and run the
GEMM inside one captured graph (torch.cuda.CUDAGraph on the capture stream),
replay it several times with eager work and synchronizations in between, and
check every replay against the eager results bit for bit.  The library queues
kernels only during a capture (no memsets, no allocation), so the whole path is
capturable; a mode (a) launch that would take the split-K schedule on a stream
without its split workspace runs unsplit instead of allocating one."""

import numpy as np
import pytest

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    import torch
    w = synth.Workload("graph", 520, 700, 1024, "a", "rowfactor_outlier", "normal", "rowwise", 41)
    XA = torch.from_numpy(synth.draw(w, "a")).cuda()
    XB = torch.from_numpy(synth.draw(w, "b")).cuda()
    M, N, K = w.M, w.N, w.K
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, device="cuda")
    sb = torch.empty(N, device="cuda")
    st = torch.empty(1, device="cuda")
    qt = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Dt = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qm = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    em = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")

    def path():
        gpu_lib.fp8_quantize_rowwise(XA, qa, sa)
        gpu_lib.fp8_quantize_rowwise(XB, qb, sb)
        gpu_lib.fp8_gemm_scaled(M, N, K, qa, qb, sa, sb, D=D)
        gpu_lib.fp8_quantize_ex(XB, per_tensor=True, q=qt, scale=st)       # clear, amax, cast, finish
        gpu_lib.fp8_gemm_scaled(M, N, K, qa, qt, sa, st.expand(N).contiguous(), D=Dt, out_dtype=torch.float32)
        gpu_lib.mxfp8_quantize(XA, qm, em)

    outs = [qa, qb, sa, sb, st, qt, D, Dt, qm, em]
    say("graph: eager")
    path()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on the side stream, as capture needs
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_() if t.dtype != torch.bfloat16 else t.fill_(7.0)
        junk = torch.randn(1 << 20, device="cuda") * 3            # eager work between replays
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(["qa", "qb", "sa", "sb", "st", "qt", "D", "Dt", "qm", "em"], outs, eager):
            assert torch.equal(t.view(torch.uint8) if t.dtype == torch.uint8 else t, e), (rep, name)
        del junk


def test_gemm_deterministic_both_tile_sizes(gpu_lib):
    """Repeated launches give identical bits, on 256x256 tiles (2561 x 3000,
    above the small-problem threshold), on 256x128 tiles (2600 x 2900) and on
    small-problem tiles (700 x 900: 64x128 in mode (a), 128x128 in mode (b)),
    in both modes."""
    import torch
    for (M, N, K) in ((2561, 3000, 1024), (2600, 2900, 1024), (700, 900, 1024)):
        A = torch.from_numpy(synth.u8_codes(51, 1, (M, K))).cuda()
        B = torch.from_numpy(synth.u8_codes(51, 2, (N, K))).cuda()
        sa = torch.rand(M, device="cuda") + 0.5
        sb = torch.rand(N, device="cuda") + 0.5
        ea = torch.from_numpy((synth.u8_codes(51, 3, (M, K // 32)) % 41 + 107).astype(np.uint8)).cuda()
        eb = torch.from_numpy((synth.u8_codes(51, 4, (N, K // 32)) % 41 + 107).astype(np.uint8)).cuda()
        say("deterministic", M, N, K)
        D1 = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
        D2 = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
        X1 = gpu_lib.mxfp8_gemm(M, N, K, A, B, ea, eb)
        X2 = gpu_lib.mxfp8_gemm(M, N, K, A, B, ea, eb)
        assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
        assert torch.equal(X1.view(torch.int16), X2.view(torch.int16))


def _split_case():
    """A mode (a) problem that takes the split-K schedule: one 128x128 tile,
    K = 4096 (32 stages) split over 4 CUs."""
    import torch
    M, N, K = 128, 128, 4096
    A = synth.u8_codes(57, 1, (M, K))
    B = synth.u8_codes(57, 2, (N, K))
    sa = (np.arange(M, dtype=np.float32) % 7 + 1) / 4
    sb = (np.arange(N, dtype=np.float32) % 5 + 1) / 8
    t = [torch.from_numpy(x).cuda() for x in (A, B, sa, sb)]
    return (M, N, K), (A, B, sa, sb), t


def test_graph_split_k_on_a_stream_with_workspace(gpu_lib):
    """Split-K launches captured on a stream that already ran one eagerly (so
    it has its split workspace): every replay equals the eager result bit for
    bit, with eager split launches on another stream in between."""
    import torch
    (M, N, K), _, (A, B, sa, sb) = _split_case()
    assert gpu_lib.fp8g_gemm_schedule(M, N, K)["split"] > 1
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)
        F = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    eager = (D.clone(), F.clone())
    g = torch.cuda.CUDAGraph()
    say("graph split-K: capture on a stream with a workspace")
    with torch.cuda.graph(g, stream=s):
        gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb, D=D)
        gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb, D=F, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for rep in range(4):
        D.fill_(7.0)
        F.zero_()
        X = gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb)      # eager split launch, current stream
        torch.cuda.synchronize()
        assert torch.equal(X.view(torch.int16), eager[0].view(torch.int16))
        say("graph split-K: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16), eager[0].view(torch.int16)), rep
        assert torch.equal(F.view(torch.int32), eager[1].view(torch.int32)), rep


def test_graph_split_k_on_a_fresh_stream(gpu_lib):
    """A split-K-sized problem captured on a stream that has no split
    workspace yet: nothing is allocated during the capture, the launch takes
    the unsplit schedule, and every replay meets the accuracy bound against
    the oracle."""
    import torch
    from gpu_util import alignment, assert_gemm_close
    from oracle import gemm
    (M, N, K), (A_h, B_h, sa_h, sb_h), (A, B, sa, sb) = _split_case()
    F = torch.empty((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    say("graph split-K: capture on a fresh stream")
    with torch.cuda.graph(g, stream=s):
        gpu_lib.fp8_gemm_scaled(M, N, K, A, B, sa, sb, D=F, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = gemm.gemm_scaled(A_h, B_h, sa_h, sb_h)
    W = gemm.gemm_scaled_weight(A_h, B_h, sa_h, sb_h)
    T = alignment(A_h, B_h, sa_h, sb_h)
    first = None
    for rep in range(3):
        F.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = F.cpu().numpy()
        assert_gemm_close(got, ref, W, "f32", "graph split-K fresh stream, replay %d" % rep, T=T)
        if first is None:
            first = got.copy()
        assert np.array_equal(got.view(np.int32), first.view(np.int32))
