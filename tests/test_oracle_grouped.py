"""Pins of the grouped spline activation oracle (``oracle/grouped.py``),
none of which re-types its formulas:

- it equals the KAN layer oracle with a block-diagonal coefficient tensor
  (O = I, C_full[j, i, m] = [j == i] C[g(i), m]): a separate code path, and the
  layer oracle is itself pinned to the pages and to textbook identities;
- dx matches central finite differences of <dy, y> in x, and dC matches the
  exact change of <dy, y> under a unit change of one coefficient (y is linear
  in C);
- on [lo, hi] the basis sums to 1, so sum_m dC[g, m] = sum of dy over the
  group's channels;
- planted mistakes (groups dealt round-robin, dy dropped from dx, B used for
  B') are each caught.
"""

import numpy as np
import pytest

import oracle
from oracle import grouped as og


def _case(N, I, groups, G, seed, spread=1.3):
    rng = np.random.default_rng(np.random.SeedSequence([31, N, I, groups, G, seed]))
    x = rng.uniform(-spread, spread, (N, I))
    C = rng.standard_normal((groups, G + 3)) * 0.3
    dy = rng.standard_normal((N, I))
    return x, C, dy


def _block_diagonal(C, I):
    groups, K = C.shape
    g = (np.arange(I) * groups) // I
    full = np.zeros((I, I, K))
    full[np.arange(I), np.arange(I)] = C[g]
    return full


@pytest.mark.parametrize("N,I,groups,G", [(7, 12, 3, 5), (5, 9, 9, 8), (6, 10, 1, 4), (4, 16, 8, 20)])
def test_equals_block_diagonal_layer(N, I, groups, G):
    x, C, dy = _case(N, I, groups, G, 0)
    full = _block_diagonal(C, I)
    y = og.grouped_forward(x, C, -1.0, 1.0, G)
    np.testing.assert_allclose(y, oracle.layer_forward(x, full, None, -1.0, 1.0, G), rtol=0, atol=1e-13)
    dx, dC = og.grouped_backward(x, C, dy, -1.0, 1.0, G)
    ldx, ldC, _ = oracle.layer_backward(x, full, None, dy, -1.0, 1.0, G)
    np.testing.assert_allclose(dx, ldx, rtol=0, atol=1e-12)
    g = (np.arange(I) * groups) // I
    want = np.zeros_like(dC)
    for i in range(I):
        want[g[i]] += ldC[i, i]
    np.testing.assert_allclose(dC, want, rtol=0, atol=1e-12)


def test_finite_differences():
    N, I, groups, G = 5, 8, 2, 6
    x, C, dy = _case(N, I, groups, G, 1)
    dx, dC = og.grouped_backward(x, C, dy, -1.0, 1.0, G)
    f = lambda xx, CC: float(np.sum(dy * og.grouped_forward(xx, CC, -1.0, 1.0, G)))
    eps = 1e-6
    for (b, i) in [(0, 0), (2, 5), (4, 7), (1, 3)]:
        xp, xm = x.copy(), x.copy()
        xp[b, i] += eps
        xm[b, i] -= eps
        assert abs((f(xp, C) - f(xm, C)) / (2 * eps) - dx[b, i]) < 1e-6
    for (g, m) in [(0, 0), (1, 4), (0, G + 2), (1, 7)]:
        Cp = C.copy()
        Cp[g, m] += 1.0
        assert abs((f(x, Cp) - f(x, C)) - dC[g, m]) < 1e-10


def test_partition_of_unity_in_dC():
    N, I, groups, G = 9, 12, 4, 8
    x, C, dy = _case(N, I, groups, G, 2, spread=0.999)
    _, dC = og.grouped_backward(x, C, dy, -1.0, 1.0, G)
    g = (np.arange(I) * groups) // I
    for gg in range(groups):
        np.testing.assert_allclose(dC[gg].sum(), dy[:, g == gg].sum(), rtol=0, atol=1e-12)


def test_group_boundaries():
    assert list(og.group_of(12, 3)) == [0] * 4 + [1] * 4 + [2] * 4
    assert list(og.group_of(5, 5)) == [0, 1, 2, 3, 4]
    assert list(og.group_of(7, 1)) == [0] * 7
    assert list(og.group_of(10, 4)) == [0, 0, 0, 1, 1, 2, 2, 2, 3, 3]


def _mutant_round_robin(x, C, dy, lo, hi, G):
    N, I = x.shape
    g = np.arange(I) % C.shape[0]
    B = oracle.basis(x, lo, hi, G)
    return np.einsum("nik,ik->ni", B, C[g])


def _mutant_dx_no_dy(x, C, dy, lo, hi, G):
    g = og.group_of(x.shape[1], C.shape[0])
    return np.einsum("nik,ik->ni", oracle.basis_derivative(x, lo, hi, G), C[g])


def _mutant_dx_with_B(x, C, dy, lo, hi, G):
    g = og.group_of(x.shape[1], C.shape[0])
    return dy * np.einsum("nik,ik->ni", oracle.basis(x, lo, hi, G), C[g])


@pytest.mark.parametrize("name", ["round_robin", "dx_no_dy", "dx_with_B"])
def test_planted_mistakes_are_caught(name):
    N, I, groups, G = 6, 12, 3, 5
    x, C, dy = _case(N, I, groups, G, 3)
    full = _block_diagonal(C, I)
    ly = oracle.layer_forward(x, full, None, -1.0, 1.0, G)
    ldx = oracle.layer_backward(x, full, None, dy, -1.0, 1.0, G)[0]
    if name == "round_robin":
        assert np.max(np.abs(_mutant_round_robin(x, C, dy, -1.0, 1.0, G) - ly)) > 1e-3
    elif name == "dx_no_dy":
        assert np.max(np.abs(_mutant_dx_no_dy(x, C, dy, -1.0, 1.0, G) - ldx)) > 1e-3
    else:
        assert np.max(np.abs(_mutant_dx_with_B(x, C, dy, -1.0, 1.0, G) - ldx)) > 1e-3
