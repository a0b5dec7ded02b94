"""concat_mla_k -- oracle, test infrastructure.

The MLA key assembly of the page on FlashInfer's concat_mla_k with FP8
inputs (sections 1-3): every key row is its 128 "nope" elements followed by
its 64 "rope" elements, 192 elements in all, for element types of 1 byte
(E4M3, E5M2) or 2 bytes (BF16, FP16).  The operation moves elements and
computes nothing, so the result is unique and checked byte for byte.

Layout read here (the page names the two parts and their widths only):
    k_nope [T, H, 128]        one row per token and head
    k_rope [T, R, 64]         R == 1: the token's rope part is shared by all
                              its heads (MLA's decoupled rotary key);
                              R == H: one rope part per head
    k      [T, H, 192]        k[t, h] = k_nope[t, h] ++ k_rope[t, 0 if R == 1 else h]
Arrays are raw element containers (uint8 for 1-byte types, uint16 for 2-byte
types): the byte patterns are copied as they are.
"""

import numpy as np

NOPE_DIM = 128
ROPE_DIM = 64
HEAD_DIM = NOPE_DIM + ROPE_DIM


def concat_mla_k(k_nope, k_rope):
    """k [T, H, 192] from k_nope [T, H, 128] and k_rope [T, R, 64], R in {1, H}."""
    k_nope = np.asarray(k_nope)
    k_rope = np.asarray(k_rope)
    if k_nope.ndim != 3 or k_nope.shape[2] != NOPE_DIM:
        raise ValueError("k_nope must be [T, H, 128]")
    T, H, _ = k_nope.shape
    if k_rope.ndim != 3 or k_rope.shape[0] != T or k_rope.shape[2] != ROPE_DIM or k_rope.shape[1] not in (1, H):
        raise ValueError("k_rope must be [T, 1, 64] or [T, H, 64]")
    if k_rope.dtype != k_nope.dtype:
        raise ValueError("k_nope and k_rope must have the same element type")
    rope = np.broadcast_to(k_rope, (T, H, ROPE_DIM))
    return np.concatenate([k_nope, rope], axis=2)
