"""Helpers for the FP8 tests: sign masks, the documented value-tile layout, dequantisation
through the oracle's e4m3 decoder (test glue only; no attention arithmetic here)."""
from __future__ import annotations

import numpy as np

import gen

TENSOR_SIGNS = 4  # generator stream of the transform's random sign mask


def sign_mask(seed):
    lo, hi = gen.words(seed, TENSOR_SIGNS, 0, 2)
    return int(lo), int(hi)


def vt_keys():
    """Key (within a 64-key tile) stored at position p of a transposed value-tile row."""
    p = np.arange(64)
    h, e = p // 32, p % 32
    return 32 * (e // 16) + 8 * ((e % 16) // 4) + 4 * h + e % 4


def vt_to_logical(vt, N_k):
    """[B,H_kv,T_c,d,64] transposed tiles -> [B,H_kv,N_k,d] codes; also returns the bytes
    stored for keys past N_k (which must be zero)."""
    B, Hk, T, d, P = vt.shape
    out = np.zeros((B, Hk, T * P, d), dtype=np.uint8)
    keys = vt_keys()
    for t in range(T):
        out[:, :, 64 * t + keys, :] = np.transpose(vt[:, :, t], (0, 1, 3, 2))
    return out[:, :, :N_k], out[:, :, N_k:]


def dequantize(orc, codes, scales, block):
    """codes [..., N, d] e4m3 with scales [..., ceil(N/block)] -> float64 values."""
    N = codes.shape[-2]
    s = np.repeat(scales.astype(np.float64), block, axis=-1)[..., :N]
    return orc.e4m3_decode(codes) * s[..., None]
