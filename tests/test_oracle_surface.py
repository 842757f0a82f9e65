"""Pins of the 2-D tensor-product spline layer oracle (``oracle/surface.py``),
none of which re-types its formula:

- textbook: scipy's ``NdBSpline`` on the same knots evaluates every edge's
  surface and its two partial derivatives, point by point;
- separable coefficients C[j,p,m,n] = a[j,p,m] * c[j,p,n] give the product of
  two 1-D splines, built from the 1-D layer oracle (a transposed C, or the
  pair's inputs swapped, fails this with a != c);
- exact reproduction on [lo, hi]^2: constant coefficients give the constant,
  and C[m,n] = xi_m * xi_n (Greville abscissae) gives x1 * x2;
- dx matches central finite differences of <dy, y>, dC the exact change of
  <dy, y> under a unit change of one coefficient;
- outside the extended grid in either input the pair contributes nothing;
- planted mistakes (C transposed in (m, n), the pair's inputs swapped, B for
  B' in the second input) are each caught.
"""

import numpy as np
import pytest
from scipy.interpolate import NdBSpline

import oracle
from oracle import surface as osf


def _case(N, P, O, G, seed, spread=1.0):
    rng = np.random.default_rng(np.random.SeedSequence([41, N, P, O, G, seed]))
    x = rng.uniform(-spread, spread, (N, 2 * P))
    C = rng.standard_normal((O, P, G + 3, G + 3)) * 0.3
    dy = rng.standard_normal((N, O))
    return x, C, dy


def _knots(lo, hi, G):
    return oracle.knots(lo, hi, G)


@pytest.mark.parametrize("G", [1, 5, 8])
def test_scipy_ndbspline(G):
    N, P, O = 9, 3, 2
    x, C, dy = _case(N, P, O, G, 0, spread=0.99)
    t = _knots(-1.0, 1.0, G)
    y = osf.surface_forward(x, C, -1.0, 1.0, G)
    dx, _ = osf.surface_backward(x, C, dy, -1.0, 1.0, G)
    want = np.zeros((N, O))
    wdx = np.zeros((N, 2 * P))
    for j in range(O):
        for p in range(P):
            s = NdBSpline((t, t), C[j, p], 3, extrapolate=False)
            pts = x[:, 2 * p:2 * p + 2]
            want[:, j] += s(pts)
            wdx[:, 2 * p] += dy[:, j] * s(pts, nu=(1, 0))
            wdx[:, 2 * p + 1] += dy[:, j] * s(pts, nu=(0, 1))
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dx, wdx, rtol=0, atol=1e-11)


def test_separable_is_product_of_1d_splines():
    N, P, O, G = 11, 4, 3, 5
    rng = np.random.default_rng(7)
    x = rng.uniform(-1.2, 1.2, (N, 2 * P))
    a = rng.standard_normal((O, P, G + 3))
    c = rng.standard_normal((O, P, G + 3))
    C = a[..., :, None] * c[..., None, :]
    y = osf.surface_forward(x, C, -1.0, 1.0, G)
    want = np.zeros((N, O))
    for j in range(O):
        for p in range(P):
            f1 = oracle.layer_forward(x[:, [2 * p]], a[j:j + 1, p:p + 1], None, -1.0, 1.0, G)[:, 0]
            f2 = oracle.layer_forward(x[:, [2 * p + 1]], c[j:j + 1, p:p + 1], None, -1.0, 1.0, G)[:, 0]
            want[:, j] += f1 * f2
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)


def test_reproduction_on_the_grid_square():
    N, P, G, lo, hi = 20, 3, 8, -1.0, 1.0
    rng = np.random.default_rng(3)
    x = rng.uniform(lo, hi, (N, 2 * P))
    K = G + 3
    ones = np.full((1, P, K, K), 2.5)
    np.testing.assert_allclose(osf.surface_forward(x, ones, lo, hi, G), np.full((N, 1), 2.5 * P),
                               rtol=0, atol=1e-12)
    xi = lo + (np.arange(K) - 1.0) * (hi - lo) / G          # Greville abscissae
    bil = np.broadcast_to(np.outer(xi, xi), (1, P, K, K))
    want = (x[:, 0::2] * x[:, 1::2]).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(osf.surface_forward(x, bil, lo, hi, G), want, rtol=0, atol=1e-12)


def test_finite_differences():
    N, P, O, G = 4, 2, 3, 6
    x, C, dy = _case(N, P, O, G, 1)
    dx, dC = osf.surface_backward(x, C, dy, -1.0, 1.0, G)
    f = lambda xx, CC: float(np.sum(dy * osf.surface_forward(xx, CC, -1.0, 1.0, G)))
    eps = 1e-6
    for (b, i) in [(0, 0), (1, 1), (3, 2), (2, 3)]:
        xp, xm = x.copy(), x.copy()
        xp[b, i] += eps
        xm[b, i] -= eps
        assert abs((f(xp, C) - f(xm, C)) / (2 * eps) - dx[b, i]) < 1e-6
    for idx in [(0, 0, 0, 0), (2, 1, 4, 7), (1, 0, 8, 2), (0, 1, 3, 3)]:
        Cp = C.copy()
        Cp[idx] += 1.0
        assert abs((f(x, Cp) - f(x, C)) - dC[idx]) < 1e-10
    # the sampled helpers equal the full computation
    rows = [0, 3]
    np.testing.assert_allclose(osf.surface_forward_rows(x, C, -1.0, 1.0, G, rows),
                               osf.surface_forward(x, C, -1.0, 1.0, G)[rows], rtol=0, atol=0)
    got = osf.surface_coef_grad_pairs(x, dy, -1.0, 1.0, G, [(2, 1), (0, 0)])
    np.testing.assert_allclose(got, dC[[2, 0], [1, 0]], rtol=0, atol=1e-13)


def test_outside_the_extended_grid_contributes_nothing():
    G = 5
    h = 2.0 / G
    x = np.array([[-1 - 3 * h - 1e-9, 0.3, 0.1, 0.2], [0.4, 1 + 3 * h, 0.1, 0.2]])
    C = np.random.default_rng(2).standard_normal((2, 2, G + 3, G + 3))
    y = osf.surface_forward(x, C, -1.0, 1.0, G)
    only2 = osf.surface_forward(x[:, 2:], C[:, 1:], -1.0, 1.0, G)
    np.testing.assert_allclose(y, only2, rtol=0, atol=1e-14)


def _mutant(kind, x, C, lo, hi, G):
    if kind == "transposed":
        return osf.surface_forward(x, np.swapaxes(C, 2, 3), lo, hi, G)
    if kind == "swapped":
        xs = x.copy()
        xs[:, 0::2], xs[:, 1::2] = x[:, 1::2], x[:, 0::2]
        return osf.surface_forward(xs, C, lo, hi, G)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["transposed", "swapped", "dx2_with_B"])
def test_planted_mistakes_are_caught(kind):
    N, P, O, G = 9, 3, 2, 5
    x, C, dy = _case(N, P, O, G, 5, spread=0.99)
    t = _knots(-1.0, 1.0, G)
    want = np.zeros((N, O))
    wdx2 = np.zeros((N, P))
    for j in range(O):
        for p in range(P):
            s = NdBSpline((t, t), C[j, p], 3, extrapolate=False)
            want[:, j] += s(x[:, 2 * p:2 * p + 2])
            wdx2[:, p] += dy[:, j] * s(x[:, 2 * p:2 * p + 2], nu=(0, 1))
    if kind == "dx2_with_B":
        B1 = oracle.basis(x[:, 0::2], -1.0, 1.0, G)
        B2 = oracle.basis(x[:, 1::2], -1.0, 1.0, G)
        bad = np.einsum("nj,npm,npq,jpmq->np", dy, B1, B2, C)
        assert np.max(np.abs(bad - wdx2)) > 1e-3
    else:
        assert np.max(np.abs(_mutant(kind, x, C, -1.0, 1.0, G) - want)) > 1e-3
