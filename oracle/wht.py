"""Walsh-Hadamard rotation over head_dim.

"spark_runtime/kv_cache.rs": ``KvCacheDtype::Turbo4`` ("Walsh-Hadamard
rotation"), ``is_wht_rotated`` (the write path rotates before quantizing;
decode applies WHT(Q) and iWHT(out) on rotated sides).

Readings (the pages give no order, normalization or signs):
  * Sylvester (natural) order, H[i][j] = (-1)^popcount(i & j), no random
    sign flips; normalized by 1/sqrt(d), so H/sqrt(d) is orthonormal and
    symmetric, hence its own inverse (the same routine is WHT and iWHT).
  * fp32 operation order on the write path: butterflies with ascending
    stride h = 1, 2, 4, ..., d/2; for every i with (i & h) == 0 the pair
    becomes (y_i + y_{i+h}, y_i - y_{i+h}), each rounded to fp32; then every
    element is multiplied once by r_d = RN32(1/sqrt(d)).
"""
from __future__ import annotations

import math

import numpy as np


def inv_sqrt_f32(d: int) -> np.float32:
    return np.float32(1.0 / math.sqrt(d))


def fwht_unnormalized_f32(y: np.ndarray) -> np.ndarray:
    """Butterflies only, fp32, ascending strides, over the last axis."""
    y = np.array(y, dtype=np.float32, copy=True)
    shape = y.shape
    d = shape[-1]
    assert d & (d - 1) == 0
    rows = y.reshape(-1, d)
    h = 1
    while h < d:
        blk = rows.reshape(rows.shape[0], d // (2 * h), 2, h)
        lo = blk[:, :, 0, :]
        hi = blk[:, :, 1, :]
        s = lo + hi            # fp32
        t = lo - hi            # fp32
        rows = np.stack([s, t], axis=2).reshape(-1, d)
        h *= 2
    return rows.reshape(shape)


def wht_f32(y: np.ndarray) -> np.ndarray:
    """Normalized rotation in fp32 with the write path's fixed operation order."""
    d = y.shape[-1]
    return fwht_unnormalized_f32(y) * inv_sqrt_f32(d)


def hadamard_f64(d: int) -> np.ndarray:
    """Orthonormal Sylvester-ordered Hadamard matrix H/sqrt(d) in fp64."""
    i = np.arange(d)
    par = np.bitwise_and(i[:, None], i[None, :])
    sign = np.ones((d, d))
    # popcount parity
    bits = par.copy()
    odd = np.zeros((d, d), dtype=bool)
    while bits.any():
        odd ^= (bits & 1).astype(bool)
        bits >>= 1
    sign[odd] = -1.0
    return sign / math.sqrt(d)
