"""Pins for the oracle's RMSNorm (the activation of the fused RMSNorm +
dequantizing GEMV, metaltile PR #250, commit adding the block-scaled fused
RMSNorm + GEMV) and for its fp64-activation matmul.

Reading pinned here (the pages give no formula): x_hat = x * g / sqrt(mean(x^2)
+ eps) per row.  Each test below fails for a plausible slip: a missing square
root, a sum in place of the mean, eps outside the root, a wrong index into g,
or one row's scale applied to another.
"""
import numpy as np
import pytest

import oracle


def _rows(seed, m=4, k=96):
    rng = np.random.default_rng(seed)
    # rows of very different magnitudes
    return (rng.standard_normal((m, k)) * np.array([1e-3, 1.0, 37.0, 2.0 ** 40])[:m, None]).astype(np.float32)


def test_unit_mean_square_without_eps():
    """g = 1, eps = 0: every normalized row has mean square exactly 1."""
    x = _rows(1)
    xh = oracle.rmsnorm(x, np.ones(x.shape[1], np.float32), 0.0)
    np.testing.assert_allclose((xh ** 2).mean(axis=1), 1.0, rtol=1e-13)


def test_closed_form_with_eps():
    """A constant row c with g = 1 normalizes to c / sqrt(c^2 + eps):
    c = 3, eps = 7 gives exactly 0.75 (eps inside the root, on the mean)."""
    x = np.full((1, 8), 3.0, np.float32)
    xh = oracle.rmsnorm(x, np.ones(8, np.float32), 7.0)
    assert (xh == 0.75).all()
    # and with g: elementwise factor
    g = np.arange(1, 9, dtype=np.float32)
    xh = oracle.rmsnorm(x, g, 7.0)
    assert (xh[0] == 0.75 * g).all()


def test_gain_is_per_element():
    """x_hat / (x * g) is one constant per row (g indexed by p, not reversed
    or shifted)."""
    rng = np.random.default_rng(2)
    x = _rows(3)
    g = rng.uniform(0.5, 2.0, x.shape[1]).astype(np.float32)
    xh = oracle.rmsnorm(x, g, 1e-6)
    ratio = xh / (x.astype(np.float64) * g.astype(np.float64))
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones_like(ratio), rtol=1e-14)


def test_scale_invariance_without_eps():
    """eps = 0: rmsnorm(4 x) == rmsnorm(x) exactly (power-of-two scaling)."""
    x = _rows(4)
    g = np.linspace(0.5, 1.5, x.shape[1], dtype=np.float32)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(x * np.float32(4.0), g, 0.0)
    assert (a == b).all()


def test_zero_row():
    x = np.zeros((2, 16), np.float32)
    assert (oracle.rmsnorm(x, np.ones(16, np.float32), 1e-6) == 0).all()
    with pytest.raises(oracle.OracleError):
        oracle.rmsnorm(x, np.ones(16, np.float32), 0.0)


def test_matmul_f64_matches_numpy():
    """The fp64-activation matmul is the plain product (numpy fp64 matmul)."""
    rng = np.random.default_rng(5)
    xh = rng.standard_normal((3, 40))
    wd = rng.standard_normal((7, 40)).astype(np.float32)
    ref, den = oracle.matmul(xh, wd)
    np.testing.assert_allclose(ref, xh @ wd.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(den, np.abs(xh) @ np.abs(wd.astype(np.float64)).T, rtol=1e-12)
