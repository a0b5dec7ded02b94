"""Build libfp8g.so (HIP, gfx950) in-tree with hipcc.

    python -m fp8_scaled_gemm_amd.build

Compiles every source under csrc/ to an object under _build/ (in parallel;
the GEMM once per operand-format pair) and links them into one shared library
next to this file.  No fast-math: the quantizer relies on IEEE fp32 division.
Packed-fp32 ops are disabled (-packed-fp32-ops); the host pass warns that it
does not know the feature, which is harmless.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8g.so")
SOURCES = ["abi.cpp", "quantize.hip", "mx_quantize.hip", "concat.hip", "roof.hip", "gemm.hip"]
# gemm.hip is compiled once per operand-format pair (FP8G_GEMM_FMT = 2 * fmt_a + fmt_b)
GEMM_PARTS = 4
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8g)")


def _units():
    """(source, extra flags, object path) for every object of the library."""
    out = []
    for src in SOURCES:
        stem = os.path.splitext(src)[0]
        if src == "gemm.hip":
            for p in range(GEMM_PARTS):
                out.append((src, ["-DFP8G_GEMM_FMT=%d" % p], os.path.join(OBJDIR, "%s_%d.o" % (stem, p))))
        else:
            out.append((src, [], os.path.join(OBJDIR, stem + ".o")))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False, jobs: int = 0) -> str:
    cc = hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    units = _units()
    cmds = [[cc] + FLAGS + extra + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            for src, extra, obj in units]
    jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(lambda c: _run(c, verbose), cmds))
    failed = [(c, out) for c, (rc, out) in zip(cmds, results) if rc != 0]
    for c, out in failed:
        sys.stderr.write(" ".join(c) + "\n" + out)
    if failed:
        raise RuntimeError("hipcc failed building libfp8g.so (%d of %d objects)" % (len(failed), len(cmds)))
    tmp = LIB + ".tmp"
    rc, out = _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [u[2] for u in units], verbose)
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("linking libfp8g.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
