"""Seeded synthetic inputs for the FP8 scaled-GEMM workloads.

This module only draws numbers: it holds none of the quantization or GEMM
arithmetic, so both the oracle side and the GPU side of a test may use it.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) in its counter form: the i-th
output of a stream with key s is mix(s + (i+1) * 0x9E3779B97F4A7C15), where
mix is the published three-step xor-shift-multiply finaliser.  Uniforms are
the top 53 bits times 2^-53; normals use the Box-Muller transform in float64
and are rounded once to float32.

The workloads follow the shapes of the ``benchmark_gemm`` runs and the
DeepGEMM call on the page "FP8 推理基础设施（五）：从 DeepGEMM 到 vLLM" and
the MXFP8 setting of the page "[sglang] FlashInfer v0.6.7 MXFP8 Gemm 통합".
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
BASE_SEED = 0xF8C0FFEE

# stream offsets within a workload
S_XA, S_XB, S_SA, S_SB, S_ROWF, S_OUTLIER, S_EA, S_EB = 1, 2, 3, 4, 5, 6, 7, 8


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    """Key of one named stream: the mixed value of seed + stream."""
    with np.errstate(over="ignore"):
        return _mix(np.array([(seed + stream) % 2**64], dtype=np.uint64))[0]


def raw_u64(key, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the stream with this key."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(key) + i * _GAMMA)


def uniform(key, start: int, count: int) -> np.ndarray:
    """float64 uniforms in [0, 1)."""
    return (raw_u64(key, start, count) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def normal(key, start: int, count: int) -> np.ndarray:
    """float64 N(0,1) draws; draw i uses stream outputs 2i and 2i+1."""
    u = uniform(key, 2 * start, 2 * count).reshape(count, 2)
    u1 = 1.0 - u[:, 0]                      # (0, 1]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u[:, 1])


_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _rows(fn, key, R, C, row0=0, chunk=1 << 18):
    """Fill an [R, C] float32 array row-major from a per-element generator
    (chunks in a thread pool; the values do not depend on the chunking)."""
    out = np.empty((R, C), dtype=np.float32)
    flat = out.reshape(-1)
    total = R * C
    base = row0 * C

    def work(s):
        n = min(chunk, total - s)
        flat[s:s + n] = fn(key, base + s, n)

    starts = range(0, total, chunk)
    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(_WORKERS) as ex:
            list(ex.map(work, starts))
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    mode: str            # "a": per-token/per-channel, "b": MXFP8
    a_recipe: str        # how the fp32 activations are drawn
    b_recipe: str
    prep: str            # "cast": raw E4M3 cast + U[0.5,2] scales; "rowwise"; "mx"
    index: int

    @property
    def seed(self) -> int:
        return BASE_SEED + 16 * self.index

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "c1_128x256x512": Workload("c1_128x256x512", 128, 256, 512, "a", "normal", "normal", "cast", 0),
    "c2_2048x1024x4096": Workload("c2_2048x1024x4096", 2048, 1024, 4096, "a", "normal", "normal", "cast", 1),
    "c3_8192x2048x8192": Workload("c3_8192x2048x8192", 8192, 2048, 8192, "a", "rowfactor", "normal002", "rowwise", 2),
    "c4_ffn_up_8192x22016x8192": Workload("c4_ffn_up_8192x22016x8192", 8192, 22016, 8192, "a", "rowfactor_outlier", "normal002", "rowwise", 3),
    "c5_mx_4096x14336x4096": Workload("c5_mx_4096x14336x4096", 4096, 14336, 4096, "b", "blockpow2", "blockpow2", "mx", 4),
}


def row_factors(seed: int, R: int, row0: int = 0) -> np.ndarray:
    """Per-row factor 10^U(-1,1) (log-uniform in [0.1, 10])."""
    return 10.0 ** (2.0 * uniform(stream_key(seed, S_ROWF), row0, R) - 1.0)


def block_pow2(seed: int, stream: int, R: int, C: int, row0: int = 0) -> np.ndarray:
    """Per-(row, 32-column block) factor 2^u, u uniform integer in [-8, 8]."""
    nb = C // 32
    u = np.floor(uniform(stream_key(seed, stream), row0 * nb, R * nb) * 17.0) - 8.0
    return np.ldexp(1.0, u.astype(np.int64)).reshape(R, nb)


def draw(w: Workload, side: str, rows: slice = None) -> np.ndarray:
    """The fp32 operand of one side ("a" -> [M,K], "b" -> [N,K]) of a workload.

    ``rows`` selects a contiguous row range so that a sample of a large
    operand can be drawn without drawing the rest (identical values).
    """
    R = w.M if side == "a" else w.N
    r0, r1, _ = (rows or slice(0, R)).indices(R)
    n = r1 - r0
    C = w.K
    recipe = w.a_recipe if side == "a" else w.b_recipe
    key = stream_key(w.seed, S_XA if side == "a" else S_XB)
    if recipe == "normal":
        return _rows(normal, key, n, C, r0)
    if recipe == "normal002":
        return _rows(lambda k, s, c: 0.02 * normal(k, s, c), key, n, C, r0)
    if recipe.startswith("rowfactor"):
        f = row_factors(w.seed, n, r0)
        outlier = recipe.endswith("outlier")
        okey = stream_key(w.seed, S_OUTLIER)
        out = np.empty((n, C), dtype=np.float32)

        def row(i):
            v = normal(key, (r0 + i) * C, C) * f[i]
            if outlier:
                v = np.where(uniform(okey, (r0 + i) * C, C) < 0.01, v * 50.0, v)
            out[i] = v

        if n > 1:
            with ThreadPoolExecutor(_WORKERS) as ex:
                list(ex.map(row, range(n)))
        else:
            for i in range(n):
                row(i)
        return out
    if recipe == "blockpow2":
        g = block_pow2(w.seed, S_EA if side == "a" else S_EB, n, C, r0)
        v = _rows(normal, key, n, C, r0).astype(np.float64)
        return (v.reshape(n, C // 32, 32) * g[:, :, None]).reshape(n, C).astype(np.float32)
    raise ValueError(recipe)


def scales(w: Workload, side: str) -> np.ndarray:
    """U[0.5, 2] fp32 per-token / per-channel scales (raw-cast workloads)."""
    R = w.M if side == "a" else w.N
    key = stream_key(w.seed, S_SA if side == "a" else S_SB)
    return (0.5 + 1.5 * uniform(key, 0, R)).astype(np.float32)


def u8_codes(seed: int, stream: int, shape, exclude_nan=True) -> np.ndarray:
    """Uniform random bytes (used as arbitrary E4M3 codes in edge-case tests)."""
    n = int(np.prod(shape))
    b = (raw_u64(stream_key(seed, stream), 0, n) >> np.uint64(56)).astype(np.uint8)
    if exclude_nan:
        b = np.where((b & 0x7F) == 0x7F, b ^ 0x01, b).astype(np.uint8)
    return b.reshape(shape)
