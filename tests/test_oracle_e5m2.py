"""Pins for the oracle's E5M2 decode and cast (CPU only).

The oracle is tied to things outside itself:
  * the OCP format table's named values (tests/golden/ocp_e5m2_values.txt);
  * torch's float8_e5m2 conversions, an independent implementation of the
    same format: decode of all 256 codes, and the cast of random fp32 bit
    patterns with |x| < 61440 (torch rounds to nearest even; from 61440 on it
    gives infinity where this cast saturates);
  * the midpoints between adjacent magnitudes, with the tie rule checked at
    each and one fp32 ulp either side.
"""

import os

import numpy as np
import torch

from oracle import e5m2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ocp_table_values():
    n = 0
    for line in open(os.path.join(GOLDEN, "ocp_e5m2_values.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = e5m2.decode_code(int(code, 16))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val), code
            assert np.signbit(got) == val.startswith("-"), code
        n += 1
    assert n == 20


def test_code_counts():
    t = e5m2.DECODE_TABLE
    assert np.isnan(t).sum() == 6 and np.isinf(t).sum() == 2
    finite = t[np.isfinite(t)]
    assert finite.size == 248 and np.unique(finite).size == 247      # +0 == -0
    scaled = finite * 65536.0                                        # multiples of 2^-16 below 2^16
    assert np.all(scaled == np.round(scaled)) and np.all(np.abs(finite) < 65536)
    assert np.array_equal(e5m2.is_finite_code(np.arange(256, dtype=np.uint8)), np.isfinite(t))


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = e5m2.DECODE_TABLE
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.all(both_nan | (ref == ours))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_roundtrip_and_monotone():
    codes = np.arange(256, dtype=np.uint8)
    fin = codes[e5m2.is_finite_code(codes)]
    assert np.array_equal(e5m2.encode(e5m2.decode(fin)), fin)
    pos = e5m2.DECODE_TABLE[:0x7C]
    assert np.all(np.diff(pos) > 0)


def test_boundary_midpoints_both_signs():
    mags = e5m2.DECODE_TABLE[:0x7C]
    for i in range(len(mags) - 1):
        mid = np.float32((mags[i] + mags[i + 1]) / 2)
        assert float(mid) == (mags[i] + mags[i + 1]) / 2          # exact in fp32
        even = i if i % 2 == 0 else i + 1
        x = np.array([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))], np.float32)
        want = np.array([even, i, i + 1], np.uint8)
        assert np.array_equal(e5m2.encode(x), want), i
        assert np.array_equal(e5m2.encode(-x), want | 0x80), i


def test_saturation_band():
    x = np.array([57344.0, 57345.0, 61439.0, 61440.0, 1e6, np.inf], dtype=np.float32)
    assert np.all(e5m2.encode(x) == 0x7B) and np.all(e5m2.encode(-x) == 0xFB)


def test_cast_matches_torch_sampled():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.abs(x) < 61440.0]
    x = np.concatenate([x, (rng.standard_normal(1 << 16) * 100).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2.encode(x), ref)
