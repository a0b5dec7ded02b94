"""GPU parity of concat_mla_k: byte-for-byte equal to the oracle
(oracle.concat.concat_mla_k), for 1-byte and 2-byte elements, shared and
per-head rope parts."""

import numpy as np
import pytest

import synth
from gpu_util import say
from oracle import concat

pytestmark = pytest.mark.gpu


def raw(seed, shape, dtype):
    bits = synth.raw_u64(synth.stream_key(seed, 1), 0, int(np.prod(shape)))
    if dtype == np.uint8:
        return (bits >> np.uint64(56)).astype(np.uint8).reshape(shape)
    return (bits >> np.uint64(48)).astype(np.uint16).reshape(shape)


# (T, H, R): single row, odd counts, shared and per-head rope, a size whose
# chunk count is not a multiple of the workgroup, and a DeepSeek-like width
CASES = [(1, 1, 1), (3, 5, 1), (3, 5, 5), (7, 16, 1), (33, 128, 1), (64, 128, 128), (257, 3, 3)]


@pytest.mark.parametrize("dtype_name", ["float8_e4m3fn", "float8_e5m2", "bfloat16", "float16"])
@pytest.mark.parametrize("T,H,R", CASES)
def test_concat_mla_k(gpu_lib, dtype_name, T, H, R):
    import torch
    tdt = getattr(torch, dtype_name)
    esz = torch.empty((), dtype=tdt).element_size()
    ndt = np.uint8 if esz == 1 else np.uint16
    nope = raw(T * 1000 + H * 10 + R, (T, H, 128), ndt)
    rope = raw(T * 1000 + H * 10 + R + 7, (T, R, 64), ndt)
    raw_t = torch.uint8 if esz == 1 else torch.int16
    dn = torch.from_numpy(nope.view(np.uint8 if esz == 1 else np.int16)).cuda().view(raw_t).view(tdt)
    dr = torch.from_numpy(rope.view(np.uint8 if esz == 1 else np.int16)).cuda().view(raw_t).view(tdt)
    say("concat_mla_k", dtype_name, T, H, R)
    k = gpu_lib.concat_mla_k(dn, dr)
    got = k.view(raw_t).cpu().numpy().view(ndt)
    want = concat.concat_mla_k(nope, rope)
    assert got.shape == want.shape
    if not np.array_equal(got, want):
        t, h, i = np.argwhere(got != want)[0]
        raise AssertionError("%d elements differ; first at (%d,%d,%d): gpu %x oracle %x"
                             % (int((got != want).sum()), t, h, i, got[t, h, i], want[t, h, i]))


def test_concat_mla_k_nan_payloads_copied(gpu_lib):
    """NaN and infinity patterns move unchanged (no value is ever computed)."""
    import torch
    nope = np.full((2, 4, 128), 0x7F, np.uint8)            # E4M3 NaN
    nope[:, :, 1::2] = 0xFF
    rope = np.full((2, 1, 64), 0x7C, np.uint8)              # E5M2 infinity pattern
    k = gpu_lib.concat_mla_k(torch.from_numpy(nope).cuda(), torch.from_numpy(rope).cuda())
    assert np.array_equal(k.cpu().numpy(), concat.concat_mla_k(nope, rope))


def test_concat_mla_k_benchmark_size(gpu_lib):
    """The concat_mla benchmark's configuration: FP8 elements, 16384 tokens x
    128 heads, one rope row shared by a token's heads; every byte of k
    compared."""
    import torch
    T, H = 16384, 128
    nope = raw(91, (T, H, 128), np.uint8)
    rope = raw(92, (T, 1, 64), np.uint8)
    say("concat_mla_k benchmark size", T, H)
    k = gpu_lib.concat_mla_k(torch.from_numpy(nope).cuda().view(torch.float8_e4m3fn),
                             torch.from_numpy(rope).cuda().view(torch.float8_e4m3fn))
    got = k.view(torch.uint8).cpu().numpy()
    del k
    assert np.array_equal(got, concat.concat_mla_k(nope, rope))
