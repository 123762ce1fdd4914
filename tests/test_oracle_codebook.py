"""Lloyd-Max codebooks pinned to the optimality conditions (evaluated by an
independent numerical integrator) and to the published Gaussian tables."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook

GOLD = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_max1960.json")


@pytest.mark.parametrize("L", [4, 8, 16])
def test_centroid_is_conditional_mean(L):
    c, t = codebook.lloyd_max_gaussian(L)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        num = integrate.quad(lambda z: z * stats.norm.pdf(z), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        den = stats.norm.cdf(b) - stats.norm.cdf(a)
        assert abs(num / den - c[k]) < 1e-10, (k, num / den, c[k])


@pytest.mark.parametrize("L", [4, 8, 16])
def test_thresholds_are_midpoints_and_symmetric(L):
    c, t = codebook.lloyd_max_gaussian(L)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    assert np.array_equal(c, -c[::-1])
    mid = t[L // 2 - 1]
    assert mid == 0.0 and not math.copysign(1.0, mid) < 0


@pytest.mark.parametrize("L", ["4", "8", "16"])
def test_matches_published_table(L):
    g = json.load(open(GOLD))
    ref = g["levels"][L]
    c, t = codebook.lloyd_max_gaussian(int(L))
    pos = c[int(L) // 2:]
    assert np.allclose(pos, ref["outputs"], rtol=0, atol=g["output_abs_tolerance"])
    mse = codebook.distortion(c, t)
    assert abs(mse - ref["mse"]) / ref["mse"] < g["mse_rel_tolerance"]


@pytest.mark.parametrize("L", [4, 8, 16])
def test_distortion_closed_form_vs_integral(L):
    c, t = codebook.lloyd_max_gaussian(L)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    mse = 0.0
    for k in range(L):
        mse += integrate.quad(lambda z: (z - c[k]) ** 2 * stats.norm.pdf(z), edges[k], edges[k + 1],
                              epsabs=1e-14)[0]
    assert abs(mse - codebook.distortion(c, t)) < 1e-11


def test_perturbing_a_centroid_raises_distortion():
    # optimality: any small move of a centroid (or threshold) increases the MSE
    for L in (4, 8, 16):
        c, t = codebook.lloyd_max_gaussian(L)
        base = codebook.distortion(c, t)
        for k in range(L):
            for d in (-1e-3, 1e-3):
                c2 = c.copy(); c2[k] += d
                assert codebook.distortion(c2, t) > base


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp32_tables(bits):
    tb = codebook.turbo_tables(bits)
    c64, t64 = tb["centroids_f64"], tb["thresholds_f64"]
    assert tb["levels"] == 1 << bits
    assert np.array_equal(tb["centroids"], c64.astype(np.float32))
    assert np.array_equal(tb["thresholds"][1:], t64.astype(np.float32))
    assert tb["inv_cmax"] == np.float32(1.0 / c64[-1])
