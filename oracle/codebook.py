"""Lloyd-Max scalar quantizers for a standard Gaussian source.

"spark_runtime/kv_cache.rs", ``KvCacheDtype::Turbo4`` doc ("Walsh-Hadamard
rotation and optimal Gaussian codebook"), ``Turbo3`` ("8 levels"),
``Turbo2`` ("4 levels").  The pages print no codebook values; the optimal
(minimum mean-squared-error) scalar quantizer of N(0,1) with L levels is the
Lloyd-Max quantizer, defined by two conditions:

  * every decision threshold is the midpoint of the two centroids beside it;
  * every centroid is the conditional mean of N(0,1) over its cell,
    (phi(a) - phi(b)) / (Phi(b) - Phi(a)) for the cell [a, b).

The fixed point is reached by alternating the two conditions (Lloyd's
method), in fp64.  The quantizer is symmetric, so the iteration runs on the
positive half (L/2 cells on [0, inf)) and mirrors it; the middle threshold is
exactly +0.0.

Tables handed to the fp32 quantizer (readings, the pages are silent):
  centroids[k]   = RN32(c_k), ascending, k = 0..L-1
  thresholds[k]  = RN32((c_{k-1} + c_k) / 2), k = 1..L-1 (index 0 unused)
  inv_cmax       = RN32(1 / c_{L-1})
"""
from __future__ import annotations

import math

import numpy as np


def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x: float) -> float:
    """Q(x) = P(Z > x) = 1 - Phi(x), accurate in the tail."""
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def lloyd_max_gaussian(levels: int, tol: float = 1e-15, settle: int = 2000,
                       max_iter: int = 100000):
    """Centroids (ascending, length L) and interior thresholds (length L-1), fp64.

    Iterates until the largest centroid update is <= `tol`, then `settle`
    more times so the result sits at the fp64 noise floor of the fixed point.
    """
    assert levels >= 2 and levels % 2 == 0
    half = levels // 2
    # start: equally spaced centroids on the positive half-line
    c = np.array([(k + 0.5) * 3.0 / half for k in range(half)], dtype=np.float64)
    for _ in range(max_iter):
        # thresholds on [0, inf): 0, midpoints, +inf
        t = np.empty(half + 1)
        t[0] = 0.0
        t[1:half] = 0.5 * (c[:-1] + c[1:])
        t[half] = math.inf
        new = np.empty(half)
        for k in range(half):
            a, b = t[k], t[k + 1]
            pa = _phi(a)
            pb = 0.0 if math.isinf(b) else _phi(b)
            mass = _upper_tail(a) - (0.0 if math.isinf(b) else _upper_tail(b))
            new[k] = (pa - pb) / mass
        delta = np.max(np.abs(new - c))
        c = new
        if delta <= tol:
            settle -= 1
            if settle < 0 or delta == 0.0:
                break
    pos = c
    centroids = np.concatenate([-pos[::-1], pos])
    thresholds = 0.5 * (centroids[:-1] + centroids[1:])
    thresholds[half - 1] = 0.0     # exactly +0.0 at the centre
    return centroids, thresholds


def turbo_tables(bits: int):
    """fp32 tables used by the turbo quantizer at `bits` bits per element."""
    L = 1 << bits
    c, t = lloyd_max_gaussian(L)
    cf = c.astype(np.float32)
    bf = np.zeros(L, dtype=np.float32)
    bf[1:] = t.astype(np.float32)
    inv_cmax = np.float32(1.0 / c[-1])
    return {"levels": L, "centroids": cf, "thresholds": bf, "inv_cmax": inv_cmax,
            "centroids_f64": c, "thresholds_f64": t}


def distortion(centroids: np.ndarray, thresholds: np.ndarray) -> float:
    """Mean-squared error of the quantizer on N(0,1) (closed form per cell)."""
    edges = np.concatenate([[-math.inf], thresholds, [math.inf]])
    mse = 0.0
    for k, ck in enumerate(centroids):
        a, b = edges[k], edges[k + 1]
        # E[(Z - c)^2 ; a<Z<b] = [Phi]_a^b (1 + c^2) + [phi*(a - 2c)] terms
        Pa = 0.0 if math.isinf(a) else 1.0 - _upper_tail(a)
        Pb = 1.0 if math.isinf(b) else 1.0 - _upper_tail(b)
        pa = 0.0 if math.isinf(a) else _phi(a)
        pb = 0.0 if math.isinf(b) else _phi(b)
        aa = 0.0 if math.isinf(a) else a * pa
        bb = 0.0 if math.isinf(b) else b * pb
        ez2 = (Pb - Pa) + (aa - bb)          # E[Z^2 ; cell]
        ez = pa - pb                         # E[Z ; cell]
        mse += ez2 - 2.0 * ck * ez + ck * ck * (Pb - Pa)
    return mse
