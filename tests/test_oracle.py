"""Pins for the float64 CPU oracle (no GPU).

Every check ties the oracle to something other than itself: invariants the
pages state (non-negativity, support of 4 intervals, the five-term truncated
power form with its [0, k+1] clamp, the quick-start shapes), textbook closed
forms (the uniform cubic pieces, exact cubic reproduction), a library
routine (SciPy's B-spline design matrix and spline derivative), brute force
(per-edge SciPy splines summed in Python loops; finite differences), and an
exact identity (the layer is linear in C and W_base).  The last test plants
plausible mistakes in copies of the oracle and shows that some pin fails.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.interpolate import BSpline

import oracle
from oracle import bspline as obs
from oracle import layer as olay

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


GRIDS = [(-1.0, 1.0, 1), (-1.0, 1.0, 5), (-1.0, 1.0, 8), (-1.0, 1.0, 20),
         (-1.0, 1.0, 50), (-2.0, 3.0, 7)]


def _xs(lo, hi, G, n=4001, outside=True):
    h = (hi - lo) / G
    a, b = (lo - 4 * h, hi + 4 * h) if outside else (lo, hi)
    xs = np.linspace(a, b, n)
    kn = obs.knots(lo, hi, G)
    xs = np.concatenate([xs, kn, kn + 0.5 * h, [lo, hi]])
    return xs if outside else xs[(xs >= lo) & (xs <= hi)]


# --------------------------------------------------------------------------
# pins as functions of the oracle callables (reused by the mutation test)
# --------------------------------------------------------------------------

def pin_partition_of_unity(basis_fn, lo, hi, G):
    x = _xs(lo, hi, G, outside=False)
    s = basis_fn(x, lo, hi, G).sum(axis=-1)
    np.testing.assert_allclose(s, 1.0, rtol=0, atol=1e-13)


def pin_truncated_power(basis_fn, lo, hi, G):
    # FlashKAN entry: five (x)_+^3 terms at shifted knots, coordinate clamped to [0, k+1]
    tp = _gold("flashkan_truncated_power.json")
    k = tp["power"]
    x = _xs(lo, hi, G)
    h = (hi - lo) / G
    t = lo + (np.arange(G + 7) - 3) * h
    ref = np.zeros(x.shape + (G + 3,))
    for m in range(G + 3):
        u = np.clip((x - t[m]) / h, tp["clamp_low"], k + tp["clamp_high_minus_degree"])
        acc = np.zeros_like(u)
        for r in range(tp["terms"]):
            acc += (-1) ** r * math.comb(4, r) * np.maximum(u - r, 0.0) ** k
        ref[:, m] = acc / math.factorial(k)
    np.testing.assert_allclose(basis_fn(x, lo, hi, G), ref, rtol=0, atol=5e-13)


def _piece(r, u):
    # textbook uniform cubic B-spline pieces (exact rationals)
    if r == 0:
        return (1 - u) ** 3 / 6
    if r == 1:
        return (3 * u ** 3 - 6 * u ** 2 + 4) / 6
    if r == 2:
        return (-3 * u ** 3 + 3 * u ** 2 + 3 * u + 1) / 6
    return u ** 3 / 6


def pin_closed_form_values(basis_fn, lo, hi, G):
    lo_f, hi_f = Fraction(lo), Fraction(hi)
    h = (hi_f - lo_f) / G
    pts, expect = [], []
    for s in range(3, G + 3):                     # spans inside [lo, hi)
        for u in (Fraction(0), Fraction(1, 4), Fraction(1, 2), Fraction(3, 4)):
            xv = lo_f + (s - 3) * h + u * h
            row = [Fraction(0)] * (G + 3)
            for r in range(4):
                row[s - 3 + r] = _piece(r, u)
            pts.append(float(xv))
            expect.append([float(v) for v in row])
    # x = hi exactly: last span, u = 0: (..., 1, 4, 1)/6 and the 4th function is 0
    row = [0.0] * (G + 3)
    row[G], row[G + 1], row[G + 2] = 1 / 6, 4 / 6, 1 / 6
    pts.append(float(hi_f))
    expect.append(row)
    got = basis_fn(np.array(pts), lo, hi, G)
    np.testing.assert_allclose(got, np.array(expect), rtol=0, atol=2e-15)


def pin_scipy_design(basis_fn, lo, hi, G):
    x = _xs(lo, hi, G, outside=False)
    x = x[(x >= lo) & (x <= hi)]
    t = lo + (np.arange(G + 7) - 3) * ((hi - lo) / G)
    dm = BSpline.design_matrix(x, t, 3).toarray()
    np.testing.assert_allclose(basis_fn(x, lo, hi, G), dm, rtol=0, atol=1e-14)


def pin_derivative_scipy(dbasis_fn, lo, hi, G, seed=0):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(G + 3)
    x = _xs(lo, hi, G, outside=False)
    x = x[(x >= lo) & (x <= hi)]
    t = lo + (np.arange(G + 7) - 3) * ((hi - lo) / G)
    d = BSpline(t, c, 3).derivative()(x)
    got = dbasis_fn(x, lo, hi, G) @ c
    np.testing.assert_allclose(got, d, rtol=0, atol=1e-11 * G)


def pin_derivative_fd(basis_fn, dbasis_fn, lo, hi, G):
    x = _xs(lo, hi, G, n=1501)
    e = 1e-6
    fd = (basis_fn(x + e, lo, hi, G) - basis_fn(x - e, lo, hi, G)) / (2 * e)
    np.testing.assert_allclose(dbasis_fn(x, lo, hi, G), fd, rtol=0, atol=2e-7 * G ** 3)


def pin_marsden(basis_fn, dbasis_fn, lo, hi, G, seed=0):
    """Exact reproduction of cubics: c_m = p(t_{m+2}) - h^2/6 p''(t_{m+2})."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(4)
    p = np.polynomial.Polynomial(a)
    h = (hi - lo) / G
    tau = lo + (np.arange(G + 3) + 2 - 3) * h
    c = p(tau) - h * h / 6 * p.deriv(2)(tau)
    x = _xs(lo, hi, G, outside=False)
    x = x[(x >= lo) & (x <= hi)]
    np.testing.assert_allclose(basis_fn(x, lo, hi, G) @ c, p(x), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dbasis_fn(x, lo, hi, G) @ c, p.deriv(1)(x), rtol=0,
                               atol=1e-10 * G)


def _tiny_layer(seed, N=6, I=3, O=2, G=5, base=True, lo=-1.0, hi=1.0, spread=1.6):
    rng = np.random.default_rng(seed)
    x = rng.uniform(lo * spread, hi * spread, (N, I))
    C = rng.standard_normal((O, I, G + 3))
    W = rng.standard_normal((O, I)) if base else None
    dy = rng.standard_normal((N, O))
    return x, C, W, dy, lo, hi, G


def pin_forward_bruteforce(fwd_fn, seed=0):
    """Per-edge SciPy splines summed in Python loops (inputs inside [lo, hi])."""
    x, C, W, dy, lo, hi, G = _tiny_layer(seed, N=5, I=4, O=3, spread=1.0)
    t = lo + (np.arange(G + 7) - 3) * ((hi - lo) / G)
    N, I = x.shape
    O = C.shape[0]
    ref = np.zeros((N, O))
    for b in range(N):
        for j in range(O):
            acc = 0.0
            for i in range(I):
                acc += float(BSpline(t, C[j, i], 3, extrapolate=False)(x[b, i]))
                acc += W[j, i] * x[b, i] / (1.0 + math.exp(-x[b, i]))
            ref[b, j] = acc
    np.testing.assert_allclose(fwd_fn(x, C, W, lo, hi, G), ref, rtol=0, atol=1e-13)


def pin_backward_fd(fwd_fn, bwd_fn, seed=0, base=True):
    """Central differences of L = <dy, y> in x, C and W_base."""
    x, C, W, dy, lo, hi, G = _tiny_layer(seed, base=base)
    dx, dC, dW = bwd_fn(x, C, W, dy, lo, hi, G)

    def L(xx, CC, WW):
        return float(np.sum(dy * fwd_fn(xx, CC, WW, lo, hi, G)))

    e = 1e-6
    fdx = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += e
        xm[idx] -= e
        fdx[idx] = (L(xp, C, W) - L(xm, C, W)) / (2 * e)
    np.testing.assert_allclose(dx, fdx, rtol=0, atol=1e-6)
    fdC = np.zeros_like(C)
    for idx in np.ndindex(*C.shape):
        Cp, Cm = C.copy(), C.copy()
        Cp[idx] += 1.0
        Cm[idx] -= 1.0
        fdC[idx] = (L(x, Cp, W) - L(x, Cm, W)) / 2.0     # exact: y is linear in C
    np.testing.assert_allclose(dC, fdC, rtol=0, atol=1e-12)
    if base:
        fdW = np.zeros_like(W)
        for idx in np.ndindex(*W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += 1.0
            Wm[idx] -= 1.0
            fdW[idx] = (L(x, C, Wp) - L(x, C, Wm)) / 2.0
        np.testing.assert_allclose(dW, fdW, rtol=0, atol=1e-12)
    else:
        assert dW is None


# --------------------------------------------------------------------------
# the pins on the oracle as committed
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_partition_of_unity(lo, hi, G):
    pin_partition_of_unity(oracle.basis, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_nonnegative_and_local_support(lo, hi, G):
    claims = _gold("inkan_claims.json")
    x = _xs(lo, hi, G)
    B = oracle.basis(x, lo, hi, G)
    assert claims["basis_nonnegative"] and B.min() >= 0.0
    t = obs.knots(lo, hi, G)
    w = claims["support_intervals"]
    for m in range(G + 3):
        outside = (x < t[m]) | (x >= t[m + w])
        assert np.all(B[outside, m] == 0.0)
    assert np.count_nonzero(B, axis=1).max() <= w
    assert B.shape[-1] == G + claims["degree"]


@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_truncated_power_form(lo, hi, G):
    pin_truncated_power(oracle.basis, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", [(-1, 1, 1), (-1, 1, 5), (-1, 1, 8), (-1, 1, 20), (-2, 3, 7)])
def test_closed_form_values(lo, hi, G):
    pin_closed_form_values(oracle.basis, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_scipy_design_matrix(lo, hi, G):
    pin_scipy_design(oracle.basis, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_derivative_vs_scipy(lo, hi, G):
    pin_derivative_scipy(oracle.basis_derivative, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", GRIDS[:5])
def test_derivative_finite_difference(lo, hi, G):
    pin_derivative_fd(oracle.basis, oracle.basis_derivative, lo, hi, G)


@pytest.mark.parametrize("lo,hi,G", GRIDS)
def test_cubic_reproduction(lo, hi, G):
    pin_marsden(oracle.basis, oracle.basis_derivative, lo, hi, G)


@pytest.mark.parametrize("G", [1, 5, 8, 20, 50])
def test_out_of_grid(G):
    lo, hi = -1.0, 1.0
    h = (hi - lo) / G
    t = obs.knots(lo, hi, G)
    x = np.array([t[0] - 1e-9, t[0] - 1.0, t[-1], t[-1] + 5.0, -1e6, 1e6])
    assert np.all(oracle.basis(x, lo, hi, G) == 0.0)
    assert np.all(oracle.basis_derivative(x, lo, hi, G) == 0.0)
    # a layer fed only such inputs reduces to the base branch, a plain matmul
    rng = np.random.default_rng(G)
    xx = rng.choice(x, size=(7, 5))
    C = rng.standard_normal((3, 5, G + 3))
    W = rng.standard_normal((3, 5))
    sil = xx / (1.0 + np.exp(-np.clip(xx, -700, 700)))
    np.testing.assert_allclose(oracle.layer_forward(xx, C, W, lo, hi, G), sil @ W.T,
                               rtol=1e-13, atol=0)
    dy = rng.standard_normal((7, 3))
    dx, dC, dW = oracle.layer_backward(xx, C, W, dy, lo, hi, G)
    assert np.all(dC == 0.0)
    dx_ref = (dy @ W) * oracle.silu_prime(xx)
    np.testing.assert_allclose(dx, dx_ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("D", [1, 3])
@pytest.mark.parametrize("G", [1, 2, 5, 8, 20, 50, 125])
def test_span_decision_near_knots(G, D):
    """The knot span is an integer decided by floating point.  The oracle's
    half-open degree-0 intervals compare x with float64 knots; the kernels take
    the largest s with fma(x, scale, shift - s) >= 0, whose sign is that of
    the exact real x * scale + shift - s for the float32 constants scale =
    G / (hi - lo) and shift = D - lo * scale.  On [-1, 1] both constants are
    exact in float32, and the two rules must pick the same span for every
    float32 input near every knot, where the degree-1 derivative jumps.  The
    kernel rule is evaluated here in exact rational arithmetic."""
    lo, hi = -1.0, 1.0
    t = obs.knots(lo, hi, G, D)
    scale = np.float32(G / (hi - lo))
    shift = np.float32(D - lo * G / (hi - lo))
    assert float(scale) == G / (hi - lo) and float(shift) == D - lo * G / (hi - lo)
    fs, fh = Fraction(float(scale)), Fraction(float(shift))
    xs = []
    for tr in t:
        f = np.float32(tr)
        for direction in (-np.inf, np.inf):
            v = f
            for _ in range(3):
                xs.append(v)
                v = np.nextafter(v, np.float32(direction))
    xs = np.unique(np.array(xs, dtype=np.float32))
    ind = obs.cox_de_boor(xs.astype(np.float64), t, 0)        # [n, G + 2D]
    inside = ind.sum(axis=1) == 1.0
    assert inside.sum() > len(t)
    for x, row, ok in zip(xs, ind, inside):
        s_kernel = math.floor(Fraction(float(x)) * fs + fh)
        if ok:
            assert s_kernel == int(np.argmax(row)), (G, D, float(x))
        else:
            assert s_kernel < 0 or s_kernel >= G + 2 * D, (G, D, float(x))


def test_silu_closed_forms():
    x = np.array([-3.0, -1.0, 0.0, 0.5, 2.0, 10.0])
    np.testing.assert_allclose(oracle.silu(x), x * (1 + np.tanh(x / 2)) / 2, rtol=1e-14)
    e = 1e-6
    fd = (oracle.silu(x + e) - oracle.silu(x - e)) / (2 * e)
    np.testing.assert_allclose(oracle.silu_prime(x), fd, atol=1e-9)
    assert oracle.silu_prime(np.array([0.0]))[0] == 0.5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_bruteforce(seed):
    pin_forward_bruteforce(oracle.layer_forward, seed)


@pytest.mark.parametrize("seed,base", [(0, True), (1, True), (2, False)])
def test_backward_finite_differences(seed, base):
    pin_backward_fd(oracle.layer_forward, oracle.layer_backward, seed, base)


def test_adjoint_identity():
    x, C, W, dy, lo, hi, G = _tiny_layer(5, N=40, I=7, O=5, G=8)
    rng = np.random.default_rng(9)
    dC_dir = rng.standard_normal(C.shape)
    dW_dir = rng.standard_normal(W.shape)
    _, dC, dW = oracle.layer_backward(x, C, W, dy, lo, hi, G)
    y0 = oracle.layer_forward(x, C, W, lo, hi, G)
    y1 = oracle.layer_forward(x, C + dC_dir, W + dW_dir, lo, hi, G)
    lhs = np.sum(dy * (y1 - y0))
    rhs = np.sum(dC * dC_dir) + np.sum(dW * dW_dir)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


def test_sampled_helpers_match_full():
    x, C, W, dy, lo, hi, G = _tiny_layer(11, N=30, I=6, O=4, G=8)
    dx, dC, dW = oracle.layer_backward(x, C, W, dy, lo, hi, G)
    y = oracle.layer_forward(x, C, W, lo, hi, G)
    rows = np.array([0, 3, 17, 29])
    np.testing.assert_allclose(oracle.layer_forward_rows(x, C, W, lo, hi, G, rows), y[rows],
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.layer_backward_rows(x, C, W, dy, lo, hi, G, rows), dx[rows],
                               rtol=1e-14, atol=1e-14)
    pairs = np.array([[0, 0], [3, 5], [2, 1], [3, 5]])
    dCp, dWp = oracle.coef_grad_pairs(x, dy, pairs, lo, hi, G, True)
    np.testing.assert_allclose(dCp, dC[pairs[:, 0], pairs[:, 1]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dWp, dW[pairs[:, 0], pairs[:, 1]], rtol=1e-13, atol=1e-13)


def test_network_chain_rule():
    rng = np.random.default_rng(3)
    lo, hi, G = -1.0, 1.0, 4
    widths = [3, 4, 2]
    layers = [(rng.standard_normal((widths[l + 1], widths[l], G + 3)) * 0.5,
               rng.standard_normal((widths[l + 1], widths[l])) * 0.5) for l in range(2)]
    x = rng.uniform(-1, 1, (5, 3))
    dy = rng.standard_normal((5, 2))
    acts = oracle.network_forward(x, layers, lo, hi, G)
    np.testing.assert_allclose(
        acts[2], oracle.layer_forward(oracle.layer_forward(x, *layers[0], lo, hi, G),
                                      *layers[1], lo, hi, G), rtol=1e-14)
    dx, grads = oracle.network_backward(acts, layers, dy, lo, hi, G)

    def L(xx, lay):
        return float(np.sum(dy * oracle.network_forward(xx, lay, lo, hi, G)[-1]))

    e = 1e-6
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += e
        xm[idx] -= e
        assert abs((L(xp, layers) - L(xm, layers)) / (2 * e) - dx[idx]) < 1e-6
    for idx in [(0, 0, 0), (1, 2, 3), (3, 1, 6)]:
        Cp = [(layers[0][0].copy(), layers[0][1]), layers[1]]
        Cm = [(layers[0][0].copy(), layers[0][1]), layers[1]]
        Cp[0][0][idx] += e
        Cm[0][0][idx] -= e
        assert abs((L(x, Cp) - L(x, Cm)) / (2 * e) - grads[0][0][idx]) < 1e-6


def test_network_bf16_cast_between_layers():
    rng = np.random.default_rng(4)
    lo, hi, G = -1.0, 1.0, 5
    layers = [(rng.standard_normal((6, 3, G + 3)), rng.standard_normal((6, 3))),
              (rng.standard_normal((2, 6, G + 3)), rng.standard_normal((2, 6)))]
    x = rng.uniform(-1, 1, (4, 3))
    acts = oracle.network_forward(x, layers, lo, hi, G, bf16_between=True)
    y1 = oracle.layer_forward(x, *layers[0], lo, hi, G)
    np.testing.assert_array_equal(acts[1], oracle.round_bf16(y1))
    np.testing.assert_allclose(acts[2], oracle.layer_forward(acts[1], *layers[1], lo, hi, G),
                               rtol=1e-15)


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0,
        np.float32(1.0) + np.arange(-300, 300, dtype=np.float32) * np.float32(2.0 ** -16),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3895314e38, np.inf, -np.inf], dtype=np.float32),
    ])
    # exact ties: mantissa low half = 0x8000
    bits = (rng.integers(0, 2 ** 15, 500, dtype=np.uint32) << 16) | 0x8000 | (0x3F << 24)
    a = np.concatenate([a, bits.view(np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a), ref)
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])


def test_quickstart_shapes():
    qs = _gold("inkan_quickstart.json")
    rng = np.random.default_rng(0)
    sl = qs["single_layer"]
    G = 8
    x = rng.uniform(-1, 1, (sl["batch"], sl["in_features"]))
    C = rng.standard_normal((sl["out_features"], sl["in_features"], G + 3))
    assert list(oracle.layer_forward(x, C, None, -1, 1, G).shape) == sl["output_shape"]
    net = qs["network"]
    w = net["widths"]
    layers = [(rng.standard_normal((w[l + 1], w[l], G + 3)) * 0.1, None) for l in range(len(w) - 1)]
    x = rng.uniform(-1, 1, (net["batch"], w[0]))
    assert list(oracle.network_forward(x, layers, -1, 1, G)[-1].shape) == net["output_shape"]


# --------------------------------------------------------------------------
# planted mistakes: each mutated copy of the oracle must fail some pin
# --------------------------------------------------------------------------

def _mut_closed_intervals(x, lo, hi, G):
    # degree-0 pieces on closed intervals [t_r, t_{r+1}]
    t = obs.knots(lo, hi, G)
    xx = np.asarray(x, dtype=np.float64)[..., None]
    B = ((t[:-1] <= xx) & (xx <= t[1:])).astype(np.float64)
    for q in range(1, 4):
        n = len(t) - q - 1
        B = ((xx - t[:n]) / (t[q:q + n] - t[:n]) * B[..., :n]
             + (t[q + 1:q + 1 + n] - xx) / (t[q + 1:q + 1 + n] - t[1:1 + n]) * B[..., 1:n + 1])
    return B


def _mut_knots_shift(x, lo, hi, G):
    # grid extended by 3 on the left only (off-by-one in the extension)
    h = (hi - lo) / G
    t = lo + (np.arange(G + 7) - 2) * h
    return obs.cox_de_boor(x, t, 3)


def _mut_deriv_sign(x, lo, hi, G):
    return -obs.basis_derivative(x, lo, hi, G)


def _mut_deriv_index(x, lo, hi, G):
    # the second (B_{m+1,k-1}) term of the derivative dropped
    t = obs.knots(lo, hi, G)
    Bl = obs.cox_de_boor(x, t, 2)
    h = (hi - lo) / G
    return Bl[..., :G + 3] / h


def _mut_fwd_transposed(x, C, W, lo, hi, G):
    # coefficient index m reversed (a transposed / flipped operand)
    return olay.layer_forward(x, C[:, :, ::-1], W, lo, hi, G)


def _mut_fwd_no_base(x, C, W, lo, hi, G):
    return olay.layer_forward(x, C, None, lo, hi, G)


def _mut_bwd_no_silu_prime(x, C, W, dy, lo, hi, G):
    dx, dC, dW = olay.layer_backward(x, C, None, dy, lo, hi, G)
    dW = None if W is None else dy.T @ olay.silu(x)
    return dx, dC, dW


def _mut_bwd_dC_transposed(x, C, W, dy, lo, hi, G):
    dx, dC, dW = olay.layer_backward(x, C, W, dy, lo, hi, G)
    return dx, dC[:, :, ::-1], dW


def _mut_bwd_dW_silu_prime(x, C, W, dy, lo, hi, G):
    dx, dC, dW = olay.layer_backward(x, C, W, dy, lo, hi, G)
    return dx, dC, (dy.T @ olay.silu_prime(x)) if W is not None else None


MUTANTS = [
    ("closed intervals", lambda: pin_partition_of_unity(_mut_closed_intervals, -1.0, 1.0, 8)),
    ("knot extension off by one", lambda: pin_scipy_design(_mut_knots_shift, -1.0, 1.0, 8)),
    ("derivative sign", lambda: pin_derivative_fd(oracle.basis, _mut_deriv_sign, -1.0, 1.0, 5)),
    ("derivative drops a term", lambda: pin_marsden(oracle.basis, _mut_deriv_index, -1.0, 1.0, 5)),
    ("forward coefficient order flipped", lambda: pin_forward_bruteforce(_mut_fwd_transposed)),
    ("forward drops the base branch", lambda: pin_forward_bruteforce(_mut_fwd_no_base)),
    ("dx drops the silu' term", lambda: pin_backward_fd(oracle.layer_forward, _mut_bwd_no_silu_prime)),
    ("dC coefficient order flipped", lambda: pin_backward_fd(oracle.layer_forward, _mut_bwd_dC_transposed)),
    ("dW uses silu' instead of silu", lambda: pin_backward_fd(oracle.layer_forward, _mut_bwd_dW_silu_prime)),
]


@pytest.mark.parametrize("name,run", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(name, run):
    with pytest.raises(AssertionError):
        run()
