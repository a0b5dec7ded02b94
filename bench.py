"""Benchmark of the FP8 scaled-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--fmt-a e4m3|e5m2] [--fmt-b e4m3|e5m2]

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM:
  ffn_up (default, 8192 x 22016 x 8192, per-token / per-channel scales):
      fp8_quantize_rowwise(X_A) -> A, sa      (activations, per token)
      fp8_quantize_rowwise(X_B) -> B, sb      (weights, per output channel)
      fp8_gemm_scaled(A, B, sa, sb) -> D      (bf16)
      with --fmt-a / --fmt-b e5m2: fp8_quantize_ex(X, fmt) to that operand's
      format and fp8_gemm_scaled_ex (default: both E4M3)
  c3 (8192 x 2048 x 8192, per-token / per-channel scales): the same three
      calls as ffn_up
  c2 (2048 x 1024 x 4096): fp8_gemm_scaled(A, B, sa, sb) -> D (bf16), on
      N(0,1) operands cast to E4M3 without scaling (cast before the timed
      region) and U[0.5, 2] scales
  mx (4096 x 14336 x 4096, MXFP8):
      mxfp8_quantize(X_A) -> A, ea            (UE8M0 per 32 K elements)
      mxfp8_quantize(X_B) -> B, eb
      mxfp8_gemm(A, B, ea, eb) -> D           (bf16)
`value` = 2 M N K / (mean step time), in TFLOP/s.  Prints one JSON line.

The line also carries
  roofline:     the GEMM kernel alone (the dominant kernel): algorithmic flops
                per launch / its mean duration from HIP events recorded on the
                launch stream over the timed region, against the dense FP8 MFMA
                peak of MI355X (5.0 PFLOP/s);
                measured_peak: the rate a roof probe reaches in the same run, right
                after the timed steps (fp8g_roof_mfma: the GEMMs' matrix-core
                instruction with no memory traffic; fp8g_roof_stream: a stream
                with the kernel's read/write mix past the infinity cache);
  cpu_baseline: the CPU oracle (numpy, float64) timed on this host on a bounded
                sample of the same workload, in the same unit.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 matrix-core peak
PEAK_HBM_GBS = 8000.0
WORKLOADS = {"ffn_up": "c4_ffn_up_8192x22016x8192", "mx": "c5_mx_4096x14336x4096",
             "c3": "c3_8192x2048x8192", "c2": "c2_2048x1024x4096",
             "concat_mla": "concat_mla_k_fp8_16384x128", "quantize": "c4_ffn_up_8192x22016x8192"}
CONCAT_T, CONCAT_H = 16384, 128     # tokens x heads, 1-byte elements, rope shared by a token's heads


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Default step counts.  After the GPU has been idle (inputs are drawn on the
# host first) its clock takes some 25-40 ms of work to ramp up: the FFN-up
# GEMM runs at about 1.36 ms per launch at first and holds 1.03 ms from about
# 40 ms on, for at least a second.  So the warmup covers about 100 ms of work
# and the timed steps about 60 ms (per mode for the quantize workload).
CONCAT_SETS = 2    # rotating buffer sets for the concat_mla workload
QUANT_SETS = 8     # rotating buffer sets for the quantize workload
DEFAULT_WARMUP = {"ffn_up": 80, "mx": 300, "c3": 500, "c2": 5000, "concat_mla": 1000, "quantize": 1000}
DEFAULT_STEPS = {"ffn_up": 50, "mx": 200, "c3": 300, "c2": 3000, "concat_mla": 500, "quantize": 500}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: about 60 ms of GPU work for the workload)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps first (default: about 100 ms of GPU work for the workload)")
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="ffn_up",
                   help="ffn_up: the FP8 GEMM path (default); c3: the same path at 8192x2048x8192; c2: the GEMM "
                        "at 2048x1024x4096 on raw-cast operands; mx: the MXFP8 path; concat_mla: concat_mla_k; "
                        "quantize: every fp8_quantize_ex mode on the FFN-up activations")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fmt-a", choices=["e4m3", "e5m2"], default="e4m3",
                   help="ffn_up: format of the activation operand A")
    p.add_argument("--fmt-b", choices=["e4m3", "e5m2"], default="e4m3",
                   help="ffn_up: format of the weight operand B")
    p.add_argument("--traffic", default=None,
                   help="counter summary with the measured HBM bytes per GEMM launch (default: the one "
                        "under profiles/ for the workload)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="only run a plain device-to-device copy of this many bytes (calibrates the "
                        "HBM byte counters of a profiler run against a known size)")
    args = p.parse_args()
    if args.steps is None:
        args.steps = DEFAULT_STEPS[args.workload]
    if args.warmup is None:
        args.warmup = DEFAULT_WARMUP[args.workload]
    return args


def copy_only(nbytes, reps=5):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes": nbytes, "seconds": dt, "GBps_read_plus_write": 2 * nbytes / dt / 1e9}))


CPU_MIN_S = 10.0   # the oracle's sample is repeated until it has run this long


def _repeat(fn, min_s=CPU_MIN_S):
    """Run fn until min_s seconds have passed: (runs, seconds)."""
    t0 = time.perf_counter()
    runs = 0
    while True:
        fn()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return runs, dt


def cpu_baseline_ffn_up(w, m_s=4096, n_s=16384, fa="e4m3", fb="e4m3"):
    """The oracle on a sample: rows 0..m_s of the activations, rows 0..n_s of the
    weights: quantize both (row-wise) and form the m_s x n_s block of D,
    repeated until CPU_MIN_S seconds have passed."""
    from oracle import gemm, quant
    XA = synth.draw(w, "a", slice(0, m_s))
    XB = synth.draw(w, "b", slice(0, n_s))

    def once():
        qa = np.empty(XA.shape, np.uint8)
        qb = np.empty(XB.shape, np.uint8)
        sa = np.empty(m_s, np.float32)
        sb = np.empty(n_s, np.float32)
        for r in range(0, m_s, 256):
            qa[r:r + 256], sa[r:r + 256] = quant.quantize_rowwise(XA[r:r + 256], fa)
        for r in range(0, n_s, 256):
            qb[r:r + 256], sb[r:r + 256] = quant.quantize_rowwise(XB[r:r + 256], fb)
        gemm.gemm_scaled(qa, qb, sa, sb, fa, fb)
    runs, dt = _repeat(once)
    flops = 2.0 * m_s * n_s * w.K * runs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "runs": runs,
            "sample": "oracle row-wise quantize of activation rows 0..%d and weight rows 0..%d, then the "
                      "%dx%dx%d block of D in float64 (numpy matmul), %d time(s); value = 2*%d*%d*%d flops "
                      "per run / time" % (m_s, n_s, m_s, n_s, w.K, runs, m_s, n_s, w.K)}


def cpu_baseline_mx(w, m_s=2048, n_s=8192):
    from oracle import gemm, quant
    XA = synth.draw(w, "a", slice(0, m_s))
    XB = synth.draw(w, "b", slice(0, n_s))

    def once():
        qa, ea = quant.mx_quantize(XA)
        qb, eb = quant.mx_quantize(XB)
        gemm.mxfp8_gemm(qa, qb, ea, eb)
    runs, dt = _repeat(once)
    flops = 2.0 * m_s * n_s * w.K * runs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "seconds": round(dt, 3), "runs": runs,
            "sample": "oracle MX quantize of rows 0..%d / 0..%d, then the %dx%dx%d block of D in float64, "
                      "%d time(s)" % (m_s, n_s, m_s, n_s, w.K, runs)}


TRAFFIC_FILES = {"ffn_up": "profiles/gemm_fp8_ffn_up_8192x22016x8192_hbm_traffic.txt",
                 "mx": "profiles/gemm_mxfp8_mx_4096x14336x4096_hbm_traffic.txt",
                 "c3": "profiles/gemm_fp8_8192x2048x8192_hbm_traffic.txt",
                 "c2": "profiles/gemm_fp8_2048x1024x4096_hbm_traffic.txt",
                 "concat_mla": "profiles/concat_mla_k_fp8_16384x128_hbm_traffic.txt",
                 "quantize": "profiles/quantize_rows_f32_e4m3_8192x8192_hbm_traffic.txt"}


def code_digest(name="gemm.hip"):
    """sha256 of a kernel source file's code, without its comments and
    whitespace: counters taken on another version of the code do not describe
    the kernel being timed, while an edit of a comment changes nothing."""
    import hashlib
    import re
    with open(os.path.join(ROOT, "fp8_scaled_gemm_amd", "csrc", name)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
    text = re.sub(r"//[^\n]*", " ", text)                 # line comments
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()


def read_traffic(path, source="gemm.hip"):
    """HBM bytes per launch of the dominant kernel from a counter summary
    ('key: value' lines), or None when the file is missing or was taken on a
    different version of the kernel's source file."""
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("code_sha256") != code_digest(source):
        log("traffic summary %s was taken on another kernel source: traffic = null" % path)
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def roof_mfma(torch, fp8g, reps=3):
    """Matrix-core roof at the current clock: the best of `reps` launches of
    fp8g_roof_mfma (two workgroups per CU, about 2 ms each), in TFLOP/s."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 8000
    flops = blocks * 4 * iters * 4 * 131072
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fp8g.fp8g_roof_mfma(blocks, iters, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return round(best, 1)


def roof_stream(torch, fp8g, write_ratio, nbytes=1 << 30, sets=2, launches=40):
    """Streaming roof: fp8g_roof_stream over `sets` distinct inputs of nbytes
    in turn (the measured kernel's own buffer geometry, past the 256 MB
    infinity cache), `launches` back to back between one event pair (as the
    streaming kernels themselves are timed), with write-back and with
    non-temporal stores (which is faster depends on whether the outputs stay
    in that cache); algorithmic bytes (read + written) per second of the
    faster policy, in GB/s."""
    srcs = [torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda") for _ in range(sets)]
    dsts = [torch.empty(nbytes // write_ratio, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    stream = torch.cuda.current_stream()
    moved = nbytes + nbytes // write_ratio
    best = 0.0
    for nt in (0, 1):
        for i in range(2 * sets):
            fp8g.fp8g_roof_stream(srcs[i % sets], dsts[i % sets], write_ratio, nt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            fp8g.fp8g_roof_stream(srcs[i % sets], dsts[i % sets], write_ratio, nt)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, moved * launches / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del srcs, dsts
    return round(best, 1)


def with_measured(roofline, measured, kind):
    roofline["measured_peak"] = measured
    roofline["measured_peak_kind"] = kind
    roofline["frac_of_measured"] = round(roofline["achieved"] / measured, 4) if measured else None
    return roofline


def concat_bench(args, torch, fp8g):
    """concat_mla_k on FP8 (1-byte) elements: k [T, H, 192] from k_nope [T, H, 128]
    and a rope part [T, 1, 64] shared by each token's heads.  value = algorithmic
    bytes (k_nope + k_rope read, k written) per second."""
    T, H = CONCAT_T, CONCAT_H
    dev = torch.device("cuda", 0)
    bits = synth.raw_u64(synth.stream_key(0xC0C0A7, 1), 0, T * H * 128 // 8)
    nope = torch.from_numpy(bits.view(np.uint8).reshape(T, H, 128)).to(dev).view(torch.float8_e4m3fn)
    bits = synth.raw_u64(synth.stream_key(0xC0C0A7, 2), 0, T * 64 // 8)
    rope = torch.from_numpy(bits.view(np.uint8).reshape(T, 1, 64)).to(dev).view(torch.float8_e4m3fn)
    k = torch.empty((T, H, 192), dtype=torch.float8_e4m3fn, device=dev)
    # calls rotate over CONCAT_SETS distinct buffer sets (671 MB each), so that
    # the 256 MB infinity cache cannot serve one call's data to the next
    sets = [(nope, rope, k)] + [(nope.clone(), rope.clone(), torch.empty_like(k)) for _ in range(CONCAT_SETS - 1)]
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        fp8g.concat_mla_k(*sets[i % CONCAT_SETS])
    torch.cuda.synchronize()
    # one event pair around the back-to-back launches on the stream (a pair per
    # 100 us launch would add its own few us)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        fp8g.concat_mla_k(*sets[i % CONCAT_SETS])
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) / args.steps * 1e3
    nbytes = T * H * 128 + T * 64 + T * H * 192
    ms = elapsed / args.steps * 1e3
    line = {"metric": "concat_mla_k GB/s (FP8, %d tokens x %d heads, rope shared)" % (T, H),
            "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": WORKLOADS["concat_mla"], "tokens": T, "heads": H, "nope": 128, "rope": 64,
                       "elem_bytes": 1, "rope_heads": 1, "rotating_buffer_sets": CONCAT_SETS,
                       "rotating_bytes": CONCAT_SETS * nbytes},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic(os.path.join(ROOT, TRAFFIC_FILES["concat_mla"]), "concat.hip"),
                         "kernel": "concat_mla_k_kernel", "bytes_per_launch": nbytes}}
    with_measured(line["roofline"], roof_stream(torch, fp8g, 1),
                  "fp8g_roof_stream: 1 GiB copy (16 bytes read, 16 written per vector), 2 rotating sets, 40 "
                  "launches back to back, the faster store policy")
    if not args.no_cpu_baseline:
        from oracle import concat
        ts = 2048                                            # tokens in the sample
        n = nope[:ts].view(torch.uint8).cpu().numpy()
        r = rope[:ts].view(torch.uint8).cpu().numpy()
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < 10.0:
            concat.concat_mla_k(n, r)
            reps += 1
        dt = (time.perf_counter() - t1) / reps
        line["cpu_baseline"] = {"value": round(ts * (H * 320 + 64) / dt / 1e9, 2), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "seconds": round(dt * reps, 2),
                                "sample": "oracle concat_mla_k (numpy) on the first %d tokens, repeated %d times"
                                          % (ts, reps)}
    print(json.dumps(line), flush=True)


QUANT_MODES = [  # (name, bf16 input, per tensor, output format)
    ("f32_row_e4m3", False, False, 0), ("bf16_row_e4m3", True, False, 0), ("f32_tensor_e4m3", False, True, 0),
    ("bf16_tensor_e4m3", True, True, 0), ("f32_row_e5m2", False, False, 1), ("bf16_row_e5m2", True, False, 1)]


def quantize_bench(args, torch, fp8g):
    """fp8_quantize_ex on the 8192 x 8192 FFN-up activations, every mode; the
    headline value is the fp32 row-wise E4M3 quantizer.  GB/s of algorithmic
    bytes: the input read (4 or 2 bytes per element), the codes written (1),
    the scales written (4 per row or 4)."""
    w = synth.WORKLOADS[WORKLOADS["quantize"]]
    dev = torch.device("cuda", 0)
    X = torch.from_numpy(synth.draw(w, "a")).to(dev)
    R, C = X.shape
    # calls rotate over QUANT_SETS distinct inputs and outputs (2.1 GB of fp32
    # input, 537 MB of codes), so that the 256 MB infinity cache can neither
    # serve one call's input to the next nor hold the codes written back
    Xs = [X] + [X.clone() for _ in range(QUANT_SETS - 1)]
    Xbs = [x.to(torch.bfloat16) for x in Xs]
    qs = [torch.empty((R, C), dtype=torch.uint8, device=dev) for _ in range(QUANT_SETS)]
    s_rows = [torch.empty((R,), dtype=torch.float32, device=dev) for _ in range(QUANT_SETS)]
    s_tens = [torch.empty((1,), dtype=torch.float32, device=dev) for _ in range(QUANT_SETS)]
    stream = torch.cuda.current_stream()
    res = {}
    for name, bf, pt, fmt in QUANT_MODES:
        xs = Xbs if bf else Xs
        scs = s_tens if pt else s_rows

        def call(i):
            j = i % QUANT_SETS
            fp8g.fp8_quantize_ex(xs[j], per_tensor=pt, q=qs[j], scale=scs[j], fmt=fmt)
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        # one event pair around the back-to-back launches on the stream: a pair
        # per launch of a 50 us kernel adds several us of its own
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        us = e0.elapsed_time(e1) / args.steps * 1e3
        nbytes = R * C * ((2 if bf else 4) + 1) + (4 if pt else 4 * R)
        res[name] = {"us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes,
                     "ms_per_call": elapsed / args.steps * 1e3}
    head = res["f32_row_e4m3"]
    line = {"metric": "fp8_quantize_ex GB/s on 8192x8192 activations (fp32 in, one scale per row, E4M3 out)",
            "value": round(head["bytes"] / (head["ms_per_call"] * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_call"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "quantize_ffn_up_activations_8192x8192", "rows": R, "cols": C,
                       "rotating_buffer_sets": QUANT_SETS, "rotating_bytes": QUANT_SETS * head["bytes"]},
            "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(head["gbs"] / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic(os.path.join(ROOT, TRAFFIC_FILES["quantize"]), "quantize.hip"),
                         "kernel": "quantize_rows_wg", "bytes_per_launch": head["bytes"]},
            "modes": {k: {"us": v["us"], "gbs": v["gbs"], "frac": round(v["gbs"] / PEAK_HBM_GBS, 4)}
                      for k, v in res.items()}}
    with_measured(line["roofline"], roof_stream(torch, fp8g, 4, R * C * 4, QUANT_SETS),
                  "fp8g_roof_stream: %d MiB read, %d MiB written per launch (the fp32 quantizer's 4:1 mix), %d "
                  "rotating sets, 40 launches back to back, the faster store policy"
                  % (R * C * 4 >> 20, R * C >> 20, QUANT_SETS))
    line["copy_roof_gbs"] = roof_stream(torch, fp8g, 1)
    if not args.no_cpu_baseline:
        from oracle import quant
        xs = X[:512].cpu().numpy()
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < 10.0:
            quant.quantize_rowwise(xs)
            reps += 1
        dt = (time.perf_counter() - t1) / reps
        line["cpu_baseline"] = {"value": round(xs.size * 5 / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "seconds": round(dt * reps, 2),
                                "sample": "oracle quantize_rowwise (numpy) on the first 512 rows, repeated %d times"
                                          % reps}
    print(json.dumps(line), flush=True)


def cpu_baseline_c2(w):
    """The oracle on the whole 2048x1024x4096 workload: cast both operands
    (E4M3, no scaling) and form D in float64."""
    from oracle import e4m3, gemm
    XA, XB = synth.draw(w, "a"), synth.draw(w, "b")
    sa, sb = synth.scales(w, "a"), synth.scales(w, "b")

    def once():
        qa, qb = e4m3.encode(XA), e4m3.encode(XB)
        gemm.gemm_scaled(qa, qb, sa, sb)
    runs, dt = _repeat(once)
    return {"value": w.flops * runs / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "seconds": round(dt, 3), "runs": runs,
            "sample": "the whole workload: oracle E4M3 cast of A and B, then all of D in float64 (numpy "
                      "matmul), %d time(s)" % runs}


def gemm_only_bench(args, torch, fp8g, w):
    """The GEMM alone on raw-cast operands (the DeepGEMM call example's
    2048x1024x4096): launches back to back between one event pair (a pair
    per 17 us launch would add its own few us)."""
    dev = torch.device("cuda", 0)
    M, N, K = w.M, w.N, w.K
    A = torch.from_numpy(synth.draw(w, "a")).to(dev).to(torch.float8_e4m3fn)   # N(0,1): no value above 448
    B = torch.from_numpy(synth.draw(w, "b")).to(dev).to(torch.float8_e4m3fn)
    sa = torch.from_numpy(synth.scales(w, "a")).to(dev)
    sb = torch.from_numpy(synth.scales(w, "b")).to(dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fp8g.fp8_gemm_scaled(M, N, K, A, B, sa, sb, D=D)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fp8g.fp8_gemm_scaled(M, N, K, A, B, sa, sb, D=D)
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) / args.steps * 1e3
    flops = float(w.flops)
    ms_per_step = elapsed / args.steps * 1e3
    achieved = flops / (us * 1e-6) / 1e12
    line = {"metric": "FP8 GEMM TFLOP/s at MxNxK=%dx%dx%d (per-token x per-channel scales, raw-cast operands)"
                      % (M, N, K),
            "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
            "data": "synthetic",
            "config": {"workload": w.name, "M": M, "N": N, "K": K, "out": "bf16",
                       "mode": "per-token x per-channel scales", "step": "gemm",
                       "operands": "N(0,1) cast to E4M3 before the timed region; scales U[0.5, 2]"},
            "kernels_us": {"gemm": round(us, 3)},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                         "traffic": read_traffic(args.traffic or os.path.join(ROOT, TRAFFIC_FILES["c2"])),
                         "kernel": "gemm_fp8_kernel", "flops_per_launch": flops}}
    with_measured(line["roofline"], roof_mfma(torch, fp8g),
                  "fp8g_roof_mfma: the scaled 32x32x64 FP8 instruction, no memory traffic, best of 3 launches")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_c2(w)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_scaled_gemm_amd as fp8g
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_only(args.copy_bytes)
        return
    fp8g.load()
    e4m3_only = args.fmt_a == "e4m3" and args.fmt_b == "e4m3"
    if not e4m3_only and args.workload != "ffn_up":
        print("--fmt-a / --fmt-b apply to the ffn_up workload only", file=sys.stderr)
        sys.exit(2)
    if args.workload == "concat_mla":
        concat_bench(args, torch, fp8g)
        return
    if args.workload == "quantize":
        quantize_bench(args, torch, fp8g)
        return
    w = synth.WORKLOADS[WORKLOADS[args.workload]]
    if w.prep == "cast":
        gemm_only_bench(args, torch, fp8g, w)
        return
    dev = torch.device("cuda", 0)

    log("drawing", w.name)
    XA = torch.from_numpy(synth.draw(w, "a")).to(dev)
    XB = torch.from_numpy(synth.draw(w, "b")).to(dev)
    M, N, K = w.M, w.N, w.K
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    if w.mode == "a":
        qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
        qb = torch.empty((N, K), dtype=torch.uint8, device=dev)
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        sb = torch.empty((N,), dtype=torch.float32, device=dev)

        fa = fp8g.FMT_E5M2 if args.fmt_a == "e5m2" else fp8g.FMT_E4M3
        fb = fp8g.FMT_E5M2 if args.fmt_b == "e5m2" else fp8g.FMT_E4M3

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            if e4m3_only:
                fp8g.fp8_quantize_rowwise(XA, qa, sa)
            else:
                fp8g.fp8_quantize_ex(XA, q=qa, scale=sa, fmt=fa)
            if ev is not None:
                ev[1].record(stream)
            if e4m3_only:
                fp8g.fp8_quantize_rowwise(XB, qb, sb)
            else:
                fp8g.fp8_quantize_ex(XB, q=qb, scale=sb, fmt=fb)
            if ev is not None:
                ev[2].record(stream)
            if e4m3_only:
                fp8g.fp8_gemm_scaled(M, N, K, qa, qb, sa, sb, D=D)
            else:
                fp8g.fp8_gemm_scaled_ex(M, N, K, qa, fa, qb, fb, sa, sb, D=D)
            if ev is not None:
                ev[3].record(stream)
        kernels = ["quantize_activations", "quantize_weights", "gemm"]
    else:
        qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
        qb = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ea = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        eb = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            fp8g.mxfp8_quantize(XA, qa, ea)
            if ev is not None:
                ev[1].record(stream)
            fp8g.mxfp8_quantize(XB, qb, eb)
            if ev is not None:
                ev[2].record(stream)
            fp8g.mxfp8_gemm(M, N, K, qa, qb, ea, eb, D=D)
            if ev is not None:
                ev[3].record(stream)
        kernels = ["quantize_activations", "quantize_weights", "gemm"]

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_kernel = {k: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
                  for j, k in enumerate(kernels)}      # microseconds
    per_kernel_median = {k: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
                         for j, k in enumerate(kernels)}

    ms_per_step = elapsed / args.steps * 1e3
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_us = per_kernel["gemm"]
    achieved = flops / (gemm_us * 1e-6) / 1e12
    # the counter summary covers the E4M3 x E4M3 kernel only
    tf = args.traffic or (os.path.join(ROOT, TRAFFIC_FILES[args.workload]) if args.workload in TRAFFIC_FILES else None)
    traffic = read_traffic(tf) if e4m3_only else None
    metric = {"ffn_up": "FP8 GEMM TFLOP/s and % of FP8 MFMA peak at MxNxK=8192x22016x8192",
              "c3": "FP8 GEMM TFLOP/s at MxNxK=8192x2048x8192 (per-token x per-channel scales)",
              "mx": "MXFP8 GEMM TFLOP/s at 4096x14336x4096"}[args.workload]
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if e4m3_only else "fp8_%s x fp8_%s" % (args.fmt_a, args.fmt_b),
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "N": N, "K": K, "out": "bf16",
                   "mode": "per-token x per-channel scales" if w.mode == "a" else "MXFP8",
                   "step": " -> ".join(kernels), "fmt_a": args.fmt_a, "fmt_b": args.fmt_b,
                   "cache": "hot: the GEMM reads the codes the step's quantizers have just written"},
        "value_basis": "2MNK / mean time of the whole step (%s); the GEMM kernel's own rate is "
                       "roofline.achieved" % " + ".join(kernels),
        "pct_of_fp8_peak_step": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "gemm_pct_of_fp8_peak": round(100.0 * achieved / PEAK_FP8_TFLOPS, 2),
        "kernels_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "kernels_us_median": {k: round(v, 2) for k, v in per_kernel_median.items()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                     "kernel": "gemm_fp8_kernel", "flops_per_launch": flops},
    }
    if w.mode == "a":
        qbytes = {"quantize_activations": M * K * 5 + 4 * M, "quantize_weights": N * K * 5 + 4 * N}
    else:   # codes + one scale byte per 32 elements
        qbytes = {"quantize_activations": M * K * 5 + M * K // 32, "quantize_weights": N * K * 5 + N * K // 32}
    line["quantizer_gbs"] = {k: round(b / (per_kernel[k] * 1e-6) / 1e9, 1) for k, b in qbytes.items()}
    with_measured(line["roofline"], roof_mfma(torch, fp8g),
                  "fp8g_roof_mfma: the scaled 32x32x64 FP8 instruction, no memory traffic, best of 3 launches")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        if w.mode == "a":
            m_s, n_s = (4096, 16384) if args.workload == "ffn_up" else (4096, w.N)
            line["cpu_baseline"] = cpu_baseline_ffn_up(w, m_s, n_s, fa=args.fmt_a, fb=args.fmt_b)
        else:
            line["cpu_baseline"] = cpu_baseline_mx(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
