"""WHT pinned to scipy's Hadamard matrix, orthonormality, involution, Parseval."""
import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import wht


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
def test_matrix_is_scipy_hadamard(d):
    assert np.array_equal(wht.hadamard_f64(d), hadamard(d) / np.sqrt(d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_butterfly_order_exact_on_integers(d):
    # small integers keep every fp32 butterfly exact, so the result must equal
    # the Sylvester-ordered matrix product exactly (pins order and signs)
    rng = np.random.default_rng(d)
    x = rng.integers(-64, 65, size=(50, d)).astype(np.float32)
    y = wht.fwht_unnormalized_f32(x)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ hadamard(d).T)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_orthonormal_and_involution(d):
    H = wht.hadamard_f64(d)
    assert np.allclose(H @ H.T, np.eye(d), atol=1e-15)
    assert np.array_equal(H, H.T)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((100, d)).astype(np.float32)
    y = wht.wht_f32(x)
    assert np.allclose(y, x.astype(np.float64) @ H.T, rtol=0, atol=2e-6 * np.abs(x).max() * np.sqrt(d) / 8)
    back = wht.wht_f32(y)
    assert np.allclose(back, x, rtol=0, atol=1e-5)
    # Parseval
    assert np.allclose((y.astype(np.float64) ** 2).sum(1), (x.astype(np.float64) ** 2).sum(1), rtol=1e-5)


def test_scale_constant():
    assert wht.inv_sqrt_f32(128).view(np.uint32) == 0x3DB504F3
    assert wht.inv_sqrt_f32(64) == np.float32(0.125)
    assert wht.inv_sqrt_f32(256) == np.float32(0.0625)
