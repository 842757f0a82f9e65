"""Pins of the oracle basis at degrees other than 3 (``oracle.basis`` /
``basis_derivative`` with ``k``), for the general-degree basis kernels:

- scipy's ``BSpline.design_matrix`` and the derivative of ``BSpline`` on the
  same extended knots, at degrees 1, 2, 4, 5;
- partition of unity and non-negativity on [lo, hi]; at most k + 1 non-zero
  functions per point;
- Marsden's identity at degree k: sum_m xi_m B_m(x) = x on [lo, hi], with the
  Greville abscissae xi_m = (t_{m+1} + ... + t_{m+k}) / k;
- the truncated-power form the FlashKAN page gives for degree k: k + 2 terms
  (-1)^i C(k+1, i) (u - i)_+^k / k!, u = (x - t_m) / h clamped to [0, k + 1];
- a planted mistake (knots extended by 3 whatever the degree) is caught.
"""

import math

import numpy as np
import pytest
from scipy.interpolate import BSpline

import oracle


def _pts(lo, hi, G, k, n=400, seed=0):
    h = (hi - lo) / G
    rng = np.random.default_rng(seed)
    return np.concatenate([rng.uniform(lo - (k + 1) * h, hi + (k + 1) * h, n),
                           lo + (np.arange(G + 2 * k + 1) - k) * h])


@pytest.mark.parametrize("k", [1, 2, 4, 5])
@pytest.mark.parametrize("G", [1, 5, 12])
def test_scipy_design_matrix_and_derivative(k, G):
    lo, hi = -1.0, 2.0
    t = oracle.knots(lo, hi, G, k)
    x = _pts(lo, hi, G, k, seed=k + G)
    # scipy's design matrix covers the base interval [t_k, t_{G+k}] = [lo, hi];
    # the extended knots beyond it are pinned by the truncated-power test
    inside = (x >= lo) & (x < hi)
    B = oracle.basis(x, lo, hi, G, k)
    D = oracle.basis_derivative(x, lo, hi, G, k)
    assert B.shape == (x.size, G + k)
    want = BSpline.design_matrix(x[inside], t, k).toarray()
    np.testing.assert_allclose(B[inside], want, rtol=0, atol=1e-12)
    assert np.all(B[(x < t[0]) | (x >= t[-1])] == 0)
    for m in range(G + k):
        c = np.zeros(G + k)
        c[m] = 1.0
        dspl = BSpline(t, c, k, extrapolate=False).derivative()
        xi = x[inside]
        # at a knot scipy may take the left piece where the oracle (half-open
        # intervals) takes the right one: compare off the knots, where both agree
        off = np.min(np.abs(xi[:, None] - t[None, :]), axis=1) > 1e-9
        np.testing.assert_allclose(oracle.basis_derivative(xi[off], lo, hi, G, k)[:, m],
                                   np.nan_to_num(dspl(xi[off])), rtol=0, atol=1e-10)
    assert np.isfinite(D).all()


@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_partition_marsden_support(k):
    lo, hi, G = -0.5, 1.5, 7
    t = oracle.knots(lo, hi, G, k)
    x = np.random.default_rng(k).uniform(lo, hi, 1000)
    B = oracle.basis(x, lo, hi, G, k)
    np.testing.assert_allclose(B.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert B.min() >= 0.0
    assert np.count_nonzero(B, axis=1).max() <= k + 1
    xi = np.array([t[m + 1:m + k + 1].mean() for m in range(G + k)])
    np.testing.assert_allclose(B @ xi, x, rtol=0, atol=1e-12)
    # derivative of Marsden's identity: sum_m xi_m B'_m(x) = 1
    np.testing.assert_allclose(oracle.basis_derivative(x, lo, hi, G, k) @ xi, 1.0, rtol=0, atol=1e-11)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_truncated_power_form(k):
    lo, hi, G = -1.0, 1.0, 6
    h = (hi - lo) / G
    t = oracle.knots(lo, hi, G, k)
    x = _pts(lo, hi, G, k, seed=10 + k)
    B = oracle.basis(x, lo, hi, G, k)
    for m in range(G + k):
        u = np.clip((x - t[m]) / h, 0.0, k + 1.0)
        tp = sum((-1) ** i * math.comb(k + 1, i) * np.maximum(u - i, 0.0) ** k for i in range(k + 2))
        np.testing.assert_allclose(tp / math.factorial(k), B[:, m], rtol=0, atol=1e-12)


def test_planted_wrong_extension_is_caught():
    lo, hi, G, k = -1.0, 1.0, 5, 2
    h = (hi - lo) / G
    t_bad = lo + (np.arange(G + 2 * 3 + 1) - 3) * h        # cubic's extension at degree 2
    x = np.random.default_rng(1).uniform(lo, hi, 50)
    bad = oracle.cox_de_boor(x, t_bad, k)
    t = oracle.knots(lo, hi, G, k)
    want = BSpline.design_matrix(x, t, k).toarray()
    assert bad.shape != want.shape or np.max(np.abs(bad - want)) > 1e-3


@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_layer_at_degree_k_per_edge(k):
    """The degree-k layer oracle against per-edge scipy splines: y[b, j] =
    sum_i BSpline(t, C[j, i], k)(x[b, i]) + W silu, and dx from the splines'
    derivatives, with x inside [lo, hi]."""
    lo, hi, G, N, I, O = -1.0, 1.0, 6, 7, 5, 3
    rng = np.random.default_rng(50 + k)
    x = rng.uniform(lo, hi, (N, I))
    C = rng.standard_normal((O, I, G + k))
    W = rng.standard_normal((O, I))
    dy = rng.standard_normal((N, O))
    t = oracle.knots(lo, hi, G, k)
    y = oracle.layer_forward(x, C, W, lo, hi, G, k=k)
    dx, dC, dW = oracle.layer_backward(x, C, W, dy, lo, hi, G, k=k)
    want = np.zeros((N, O))
    wdx = np.zeros((N, I))
    for j in range(O):
        for i in range(I):
            s = BSpline(t, C[j, i], k)
            want[:, j] += s(x[:, i]) + W[j, i] * oracle.silu(x[:, i])
            wdx[:, i] += dy[:, j] * (s.derivative()(x[:, i]) + W[j, i] * oracle.silu_prime(x[:, i]))
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dx, wdx, rtol=0, atol=1e-10)
    # dC: the exact change of <dy, y> under a unit change of one coefficient
    f = lambda CC: float(np.sum(dy * oracle.layer_forward(x, CC, W, lo, hi, G, k=k)))
    for idx in [(0, 0, 0), (2, 4, G + k - 1), (1, 2, 3)]:
        Cp = C.copy()
        Cp[idx] += 1.0
        assert abs(f(Cp) - f(C) - dC[idx]) < 1e-10
