"""Pins for the oracle's E4M3FN decode and cast (CPU only).

The oracle is tied to things outside itself:
  * the OCP format table (tests/golden/ocp_e4m3_values.txt) and the pages' 448;
  * torch's own float8_e4m3fn conversions, an independent implementation of
    the same format: decode of all 256 codes, and the cast of every fp32 bit
    pattern with |x| <= 464 (torch rounds to nearest-even there; above 464 it
    gives NaN where this library saturates);
  * the boundary midpoints between adjacent magnitudes, derived here from the
    bit definition, with the tie rule checked at each and one fp32 ulp either side.
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (t.strip() for t in line.split("=", 1))
            out[k] = v
    return out


def test_page_max_is_448():
    facts = _read_kv("pages_facts.txt")
    assert float(facts["e4m3_max"]) == 448.0
    finite = e4m3.DECODE_TABLE[~np.isnan(e4m3.DECODE_TABLE)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_ocp_table_values():
    for line in open(os.path.join(GOLDEN, "ocp_e4m3_values.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = e4m3.decode_code(int(code, 16))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val), code
            assert np.signbit(got) == val.startswith("-"), code


def test_code_counts():
    t = e4m3.DECODE_TABLE
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    finite = t[~np.isnan(t)]
    assert finite.size == 254
    assert np.unique(finite).size == 253            # +0 and -0 compare equal
    # every finite value is an integer multiple of 2^-9, below 2^9
    scaled = finite * 512.0
    assert np.all(scaled == np.round(scaled)) and np.all(np.abs(finite) < 512)


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))
    assert np.all(np.signbit(ref[~both_nan]) == np.signbit(ours[~both_nan]))


def test_roundtrip_and_monotone():
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([e4m3.decode_code(c) for c in finite], dtype=np.float32)
    assert np.array_equal(e4m3.encode(vals), np.array(finite, dtype=np.uint8))
    mags = e4m3.DECODE_TABLE[:0x7F]
    assert np.all(np.diff(mags) > 0)


def _midpoint_cases():
    """(x, expected code) from the bit definition: each midpoint between
    adjacent magnitudes goes to the even code; one fp32 ulp below goes down,
    one above goes up.  The last midpoint, 464, lies between 448 (0x7E, even)
    and the first value past the top (480, which would be the NaN pattern):
    it and everything above saturate to 0x7E."""
    cases = []
    for lo in range(0x7E):
        hi = lo + 1
        a, b = e4m3.decode_code(lo), e4m3.decode_code(hi)
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2                 # exact in fp32
        even = lo if lo % 2 == 0 else hi
        cases.append((mid, even))
        cases.append((np.nextafter(mid, np.float32(0)), lo))
        cases.append((np.nextafter(mid, np.float32(np.inf)), hi))
    m = np.float32(464.0)
    cases += [(m, 0x7E), (np.nextafter(m, np.float32(0)), 0x7E),
              (np.nextafter(m, np.float32(np.inf)), 0x7E), (np.float32(1e30), 0x7E),
              (np.float32(np.inf), 0x7E)]
    return cases


def test_boundary_midpoints_both_signs():
    cases = _midpoint_cases()
    assert len(cases) == 126 * 3 + 5
    x = np.array([c[0] for c in cases], dtype=np.float32)
    want = np.array([c[1] for c in cases], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(x), want)
    assert np.array_equal(e4m3.encode(-x), want | 0x80)


def test_named_rounding_examples():
    # ties: 2^-10 -> 0 (even), 3*2^-10 -> 2, 15*2^-10 (between 0x07 and 0x08) -> 0x08
    x = np.array([2 ** -10, 3 * 2 ** -10, 15 * 2 ** -10, -1e-30, -0.0, 0.0], dtype=np.float32)
    assert list(e4m3.encode(x)) == [0x00, 0x02, 0x08, 0x80, 0x80, 0x00]
    assert e4m3.encode(np.float32(np.nan)) & 0x7F == 0x7F


def test_saturation_band():
    x = np.array([448.0, 449.0, 463.99, 464.0, 464.01, 479.0, 480.0, 1e6, 3.4e38], dtype=np.float32)
    assert np.all(e4m3.encode(x) == 0x7E)
    assert np.all(e4m3.encode(-x) == 0xFE)


def _torch_cast(x):
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_cast_matches_torch_sampled():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    keep = np.abs(x) <= 464.0                     # torch's range of agreement (NaNs excluded)
    x = x[keep]
    assert np.array_equal(e4m3.encode(x), _torch_cast(x))


@pytest.mark.slow
def test_cast_matches_torch_exhaustive():
    """Every positive fp32 pattern up to 464 (1.14e9 values), and the sign
    rule on a 1-in-64 stride of them."""
    top = int(np.array([464.0], dtype=np.float32).view(np.uint32)[0])
    chunk = 1 << 20
    for start in range(0, top + 1, chunk):
        stop = min(start + chunk, top + 1)
        x = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        ours = e4m3.encode(x)
        ref = _torch_cast(x)
        if not np.array_equal(ours, ref):
            bad = np.nonzero(ours != ref)[0][0]
            raise AssertionError("mismatch at bits 0x%08x: oracle %02x torch %02x"
                                 % (start + bad, ours[bad], ref[bad]))
        if (start // chunk) % 64 == 0:
            assert np.array_equal(e4m3.encode(-x), ours | 0x80)
