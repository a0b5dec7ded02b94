"""Pins for the oracle's concat_mla_k (CPU only): an element-by-element loop
written from the row definition (128 nope elements, then 64 rope elements),
and element values that encode their own source position."""

import numpy as np
import pytest

from oracle import concat


def brute(k_nope, k_rope):
    T, H, _ = k_nope.shape
    R = k_rope.shape[1]
    out = np.zeros((T, H, 192), k_nope.dtype)
    for t in range(T):
        for h in range(H):
            for i in range(192):
                out[t, h, i] = k_nope[t, h, i] if i < 128 else k_rope[t, 0 if R == 1 else h, i - 128]
    return out


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("T,H,R", [(1, 1, 1), (3, 4, 1), (2, 5, 5), (4, 2, 2)])
def test_matches_elementwise_loop(dtype, T, H, R):
    rng = np.random.default_rng(T * 100 + H * 10 + R)
    hi = 256 if dtype == np.uint8 else 65536
    k_nope = rng.integers(0, hi, (T, H, 128)).astype(dtype)
    k_rope = rng.integers(0, hi, (T, R, 64)).astype(dtype)
    assert np.array_equal(concat.concat_mla_k(k_nope, k_rope), brute(k_nope, k_rope))


def test_positions_encoded_in_values():
    # 16-bit elements carrying (token, head, index) so that any misplaced
    # element is identified by its value
    T, H = 3, 4
    t, h, i = np.meshgrid(np.arange(T), np.arange(H), np.arange(128), indexing="ij")
    k_nope = (t * 4096 + h * 256 + i).astype(np.uint16)
    tr, ir = np.meshgrid(np.arange(T), np.arange(64), indexing="ij")
    k_rope = (40000 + tr * 64 + ir).astype(np.uint16)[:, None, :]
    k = concat.concat_mla_k(k_nope, k_rope)
    assert k.shape == (T, H, 192)
    for tt in range(T):
        for hh in range(H):
            assert list(k[tt, hh, :128]) == [tt * 4096 + hh * 256 + j for j in range(128)]
            assert list(k[tt, hh, 128:]) == [40000 + tt * 64 + j for j in range(64)]


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        concat.concat_mla_k(np.zeros((2, 3, 127), np.uint8), np.zeros((2, 1, 64), np.uint8))
    with pytest.raises(ValueError):
        concat.concat_mla_k(np.zeros((2, 3, 128), np.uint8), np.zeros((2, 2, 64), np.uint8))
    with pytest.raises(ValueError):
        concat.concat_mla_k(np.zeros((2, 3, 128), np.uint8), np.zeros((2, 1, 64), np.uint16))
