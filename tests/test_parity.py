"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Tolerances: float32 path, normwise max relative error <= 1e-5 per output
tensor; bf16-input / float32-accumulate path, relative Frobenius error <= 1e-2
per output tensor.  Small shapes are compared element by element in full;
the full-size workloads are compared on seeded samples of rows (y, dx: a row
depends only on the same row of the inputs) and of (j, i) pairs (dC, dW: each
entry is its own sum over all rows), which the oracle computes one by one.
"""

import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from kan_testutil import TOL_BF16, TOL_F32, ensure_built, metric, rel_fro, rel_inf, to_dev

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def F():
    ensure_built()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kolmogorov_arnold_network_amd import functional
    return functional


def _sync():
    import torch
    torch.cuda.synchronize()


def _np(t):
    return None if t is None else t.detach().float().cpu().numpy()


# ---------------------------------------------------------------------------
# basis step alone
@pytest.mark.parametrize("G", [1, 5, 8, 20, 50])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_basis_kernel(F, G, dtype):
    claims = json.load(open(os.path.join(GOLD, "inkan_claims.json")))
    lo, hi = -1.0, 1.0
    h = (hi - lo) / G
    rng = np.random.default_rng(G)
    x = np.concatenate([rng.uniform(lo - 4 * h, hi + 4 * h, 200000),
                        lo + (np.arange(G + 7) - 3) * h, [lo, hi, 0.0, lo - 1e-7, hi + 1e-7]])
    x = x.astype(np.float32)
    if dtype == "bf16":
        x = wl.to_bf16_values(x)
    say("basis G=%d dtype=%s n=%d" % (G, dtype, x.size))
    B, dB = F.kan_basis_eval(to_dev(x, dtype), (lo, hi, G))
    _sync()
    B, dB = _np(B), _np(dB)
    ref = oracle.basis(x.astype(np.float64), lo, hi, G)
    dref = oracle.basis_derivative(x.astype(np.float64), lo, hi, G)
    tol = 2 * claims["basis_float32_abs_accuracy"]
    assert np.max(np.abs(B - ref)) <= tol
    assert B.min() >= 0.0                                    # non-negative, bitwise
    assert np.count_nonzero(B, axis=1).max() <= claims["support_intervals"]
    assert np.max(np.abs(dB - dref)) <= tol * 4 * (G / (hi - lo))


# Truncated-power form (FlashKAN page): (u^3 - 4 (u-1)_+^3 + 6 (u-2)_+^3 -
# 4 (u-3)_+^3) / 6 with u clamped to [0, 4].  Error bound in float32: the
# four terms' magnitudes sum to at most (64 + 4*27 + 6*8 + 4) / 6 = 37.3,
# each carrying ~2 roundings, and the three partial sums (<= 64) one each:
# ~107 ulp of 1, 6.4e-6 -> tolerance 1e-5.  The derivative in units of 1/h:
# (16 + 4*9 + 6*4 + 4) / 2 = 40 and partial sums <= 16: ~64 ulp, 3.8e-6.
TP_TOL = 1e-5


@pytest.mark.parametrize("G", [1, 5, 8, 20, 50])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_basis_truncated_power(F, G, dtype):
    lo, hi = -1.0, 1.0
    h = (hi - lo) / G
    rng = np.random.default_rng(100 + G)
    x = np.concatenate([rng.uniform(lo - 4 * h, hi + 4 * h, 200000),
                        lo + (np.arange(G + 7) - 3) * h, [lo, hi, 0.0, lo - 1e-7, hi + 1e-7, -50.0, 50.0]])
    x = x.astype(np.float32)
    if dtype == "bf16":
        x = wl.to_bf16_values(x)
    say("truncated-power basis G=%d dtype=%s n=%d" % (G, dtype, x.size))
    xt = to_dev(x, dtype)
    B, dB = F.kan_basis_eval_tp(xt, (lo, hi, G))
    Bl, _ = F.kan_basis_eval(xt, (lo, hi, G), need_dB=False)
    _sync()
    B, dB, Bl = _np(B), _np(dB), _np(Bl)
    ref = oracle.basis(x.astype(np.float64), lo, hi, G)
    dref = oracle.basis_derivative(x.astype(np.float64), lo, hi, G)
    e, el = np.max(np.abs(B - ref)), np.max(np.abs(Bl - ref))
    ed = np.max(np.abs(dB - dref)) * h
    say("  max |B - B_exact|: truncated power %.2e, local span %.2e; min B %.2e; "
        "max |dB - dB_exact| h %.2e" % (e, el, B.min(), ed))
    assert e <= TP_TOL and ed <= TP_TOL
    # exactly zero beyond the extended grid and far outside it (the test in
    # float64: the float32 knot t_{G+6} may lie just inside the grid)
    xd = x.astype(np.float64)
    far = (xd < lo - 3 * h) | (xd >= hi + 3 * h)
    assert np.all(B[far] == 0.0) and np.all(dB[far] == 0.0)



# Degrees 1, 2, 4, 5 (the basis step only; the layer is cubic).  Tolerances
# from the arithmetic: the local recurrence adds non-negative terms, about
# 2 D roundings of values <= 1, so 2e-6 (dB in units of 1/h likewise).  The
# truncated-power sum has terms of total size S_D = sum_i C(D+1, i)
# (D+1-i)^D / D! (4, 27, 37.3, 120, 394 for D = 1 .. 5), each carrying about
# 2 roundings: 4 S_D ulp of 1.  Its derivative's terms, in units of 1/h, total
# D S_{D-1}-like sums; the same bound with the degree-(D-1) powers is used.
def _tp_scale(D, power):
    import math
    return sum(math.comb(D + 1, i) * (D + 1 - i) ** power for i in range(D + 2)) / math.factorial(power)


@pytest.mark.parametrize("D", [1, 2, 4, 5])
@pytest.mark.parametrize("G", [1, 5, 20, 125])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_basis_general_degree(F, D, G, dtype):
    lo, hi = -1.0, 1.0
    h = (hi - lo) / G
    rng = np.random.default_rng(100 * D + G)
    x = np.concatenate([rng.uniform(lo - (D + 1) * h, hi + (D + 1) * h, 100000),
                        lo + (np.arange(G + 2 * D + 1) - D) * h, [lo, hi, 0.0]]).astype(np.float32)
    if dtype == "bf16":
        x = wl.to_bf16_values(x)
    say("basis degree %d G=%d %s n=%d" % (D, G, dtype, x.size))
    ref = oracle.basis(x.astype(np.float64), lo, hi, G, D)
    dref = oracle.basis_derivative(x.astype(np.float64), lo, hi, G, D) * h
    B, dB = F.kan_basis_eval(to_dev(x, dtype), (lo, hi, G), degree=D)
    B, dB = _np(B), _np(dB) * h
    assert B.shape == ref.shape
    assert np.max(np.abs(B - ref)) <= 2e-6 and np.max(np.abs(dB - dref)) <= 2e-6 * (D + 1)
    assert B.min() >= 0.0
    assert np.count_nonzero(B, axis=1).max() <= D + 1
    Bt, dBt = F.kan_basis_eval_tp(to_dev(x, dtype), (lo, hi, G), degree=D)
    Bt, dBt = _np(Bt), _np(dBt) * h
    eps = 2.0 ** -24
    assert np.max(np.abs(Bt - ref)) <= 4 * eps * _tp_scale(D, D) + 1e-7
    assert np.max(np.abs(dBt - dref)) <= 4 * eps * (D + 1) * _tp_scale(D, max(D - 1, 0)) + 1e-7

# ---------------------------------------------------------------------------
# small ragged layers, every variant, in full
SMALL = [  # N, I, O, G, base
    (1, 1, 1, 1, True), (37, 5, 3, 8, False), (300, 29, 17, 5, True), (513, 64, 260, 20, True),
    (100, 13, 7, 50, False), (257, 40, 300, 8, True), (64, 256, 31, 3, True), (20, 3, 513, 12, False),
    (40, 5, 70, 125, True),     # the largest grid: K = 128, the gather kernels' LDS bound
    # gather forward: 1024-thread blocks (K > 32) with the inputs split in
    # 8 slices; 64-row blocks split in 32 slices of 8 inputs with a ragged tail
    (600, 64, 100, 40, True), (70, 250, 66, 8, False),
]


def _layer_on_gpu(F, d, variant):
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    dt = d["dtype"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt, dyt = to_dev(x, dt), to_dev(C, dt), to_dev(W, dt), to_dev(dy, "f32")
    y = F.kan_forward(xt, Ct, Wt, grid, variant)
    dx, dC, dW = F.kan_backward(xt, Ct, Wt, dyt, grid, variant=variant)
    _sync()
    return _np(y), _np(dx), _np(dC), _np(dW)


def _layer_oracle(d):
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    y = oracle.layer_forward(x, C, W, *grid)
    dx, dC, dW = oracle.layer_backward(x, C, W, dy, *grid)
    return y, dx, dC, dW


@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["mfma", "gather"])
def test_small_layer(F, shape, dtype, variant):
    N, I, O, G, base = shape
    say("small layer %s dtype=%s variant=%s" % (shape, dtype, variant))
    d = wl.random_layer(N, I, O, G, dtype=dtype, base=base, seed=N + I + O + G)
    got = _layer_on_gpu(F, d, variant)
    ref = _layer_oracle(d)
    err, tol = metric(dtype)
    for name, a, r in zip(("y", "dx", "dC", "dW"), got, ref):
        if r is None:
            assert a is None
            continue
        e = err(a, r)
        assert e <= tol, "%s error %.3e > %.0e" % (name, e, tol)


# bf16 layers whose forward runs on the 2:4-sparse matrix instructions:
# N, I, O, G, base (columns per input Kb -> groups NG)
SPARSE = [
    (300, 37, 70, 7, True),     # Kb 11 -> NG 4
    (129, 50, 33, 12, False),   # Kb 15 -> NG 4
    (77, 23, 260, 17, True),    # Kb 21 -> NG 6
    (256, 66, 40, 20, True),    # Kb 24 -> NG 6, inputs straddle k-tiles
    (45, 9, 19, 21, False),     # Kb 24 -> NG 6, no base branch
    (300, 31, 50, 28, True),    # Kb 32 -> NG 8
    (70, 17, 24, 26, False),    # Kb 29 -> NG 8
]


# Layers of spline degree D != 3 (the FlashKAN page's degree-k basis): both
# passes on the matrix cores, against the degree-D oracle; the layer's
# tolerances.
DEG_CASES = [(70, 29, 33, 8, 1), (70, 29, 33, 8, 2), (50, 40, 17, 5, 4), (40, 13, 300, 20, 5), (33, 9, 5, 1, 4),
             # the largest grid: 126 (degree 1) and 130 (degree 5) coefficients per edge
             (19, 4, 5, 125, 1), (21, 3, 7, 125, 5)]


@pytest.mark.parametrize("N,I,O,G,D", DEG_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("base", [True, False])
@pytest.mark.parametrize("variant", ["auto", "mfma", "gather"])
def test_layer_general_degree(F, N, I, O, G, D, dtype, base, variant):
    say("degree-%d layer %dx(%d->%d) G=%d %s base=%s variant=%s" % (D, N, I, O, G, dtype, base, variant))
    d = wl.random_layer(N, I, O, G, dtype=dtype, base=base, seed=D, degree=D)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], G)
    xt, Ct, Wt, dyt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype), to_dev(dy, "f32")
    y = F.kan_forward(xt, Ct, Wt, grid, variant)
    dx, dC, dW = F.kan_backward(xt, Ct, Wt, dyt, grid, variant=variant)
    ry = oracle.layer_forward(x, C, W, *grid, k=D)
    rdx, rdC, rdW = oracle.layer_backward(x, C, W, dy, *grid, k=D)
    err, tol = metric(dtype)
    assert err(_np(y), ry) <= tol
    assert err(_np(dx), rdx) <= tol
    assert err(_np(dC), rdC) <= tol
    if base:
        assert err(_np(dW), rdW) <= tol


@pytest.mark.parametrize("shape", SPARSE, ids=["x".join(map(str, s)) for s in SPARSE])
def test_sparse_forward(F, shape):
    """The structured-sparse forward against the oracle, and against the
    dense forward on the same stored bits (the same bf16 products summed in
    float32 in another order)."""
    N, I, O, G, base = shape
    say("sparse forward %s" % (shape,))
    d = wl.random_layer(N, I, O, G, dtype="bf16", base=base, seed=3 * N + I + O + G)
    (C, W), x = d["layers"][0], d["x"]
    grid = (d["lo"], d["hi"], G)
    xt, Ct, Wt = to_dev(x, "bf16"), to_dev(C, "bf16"), to_dev(W, "bf16")
    y_s = F.kan_forward(xt, Ct, Wt, grid, "mfma")
    y_d = F.kan_forward(xt, Ct, Wt, grid, "mfma", dense_forward=True)
    _sync()
    y_s, y_d = _np(y_s), _np(y_d)
    ref = oracle.layer_forward(x, C, W, *grid)
    assert rel_fro(y_s, ref) <= TOL_BF16
    assert rel_inf(y_s, y_d) <= 1e-5


# Truncated-power forward generator: the SPARSE shapes plus the two bf16
# workloads' grids (G = 5: 9 columns per input; G = 20: 24).
TP_CASES = SPARSE + [(300, 40, 70, 5, True), (129, 70, 33, 20, True)]


@pytest.mark.parametrize("shape", TP_CASES, ids=["x".join(map(str, s)) for s in TP_CASES])
def test_tp_forward(F, shape):
    """The dense forward with its operand built from truncated powers, against
    the oracle at the bf16 bar and against the span-based dense forward (the
    two round different float32 basis values to bf16)."""
    N, I, O, G, base = shape
    say("truncated-power forward %s" % (shape,))
    d = wl.random_layer(N, I, O, G, dtype="bf16", base=base, seed=5 * N + I + O + G)
    (C, W), x = d["layers"][0], d["x"]
    grid = (d["lo"], d["hi"], G)
    xt, Ct, Wt = to_dev(x, "bf16"), to_dev(C, "bf16"), to_dev(W, "bf16")
    y_t = F.kan_forward(xt, Ct, Wt, grid, "mfma", tp_forward=True)
    y_d = F.kan_forward(xt, Ct, Wt, grid, "mfma", dense_forward=True)
    _sync()
    y_t, y_d = _np(y_t), _np(y_d)
    ref = oracle.layer_forward(x, C, W, *grid)
    assert rel_fro(y_t, ref) <= TOL_BF16
    assert rel_fro(y_t, y_d) <= TOL_BF16


def test_deterministic_and_prepared(F):
    import torch
    d = wl.random_layer(700, 48, 300, 8, dtype="bf16", base=True, seed=5)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt, dyt = to_dev(x, "bf16"), to_dev(C, "bf16"), to_dev(W, "bf16"), to_dev(dy, "f32")
    say("determinism bf16 700x48x300")
    outs = []
    for _ in range(3):
        outs.append((F.kan_forward(xt, Ct, Wt, grid, "mfma"),) +
                    F.kan_backward(xt, Ct, Wt, dyt, grid, variant="mfma"))
    _sync()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)
    # pre-packed workspaces give the same bits
    from kolmogorov_arnold_network_amd import _lib as L
    wsf = F.kan_prepare(xt, Ct, Wt, grid, L.KAN_PASS_FORWARD, variant="mfma")
    y2 = F.kan_forward(xt, Ct, Wt, grid, "mfma", ws=wsf, prepared=True)
    wsb = F.kan_prepare(xt, Ct, Wt, grid, L.KAN_PASS_BACKWARD, dy=dyt, variant="mfma")
    b2 = F.kan_backward(xt, Ct, Wt, dyt, grid, variant="mfma", ws=wsb, prepared=True)
    _sync()
    assert torch.equal(y2, outs[0][0])
    for a, b in zip(b2, outs[0][1:]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_batch_dc(F, dtype):
    """2048 rows against 2 output tiles: dC runs in 4 (bf16) or 8 (float32)
    fixed batch slices that are summed in slice order (no atomics).  dC
    alone, dW_base alone and both together give the oracle's values and the
    same bits, every time.  The G = 20 bf16 layer also takes the 2:4 sparse
    forward (the SPARSE shapes above cover its k-split)."""
    import torch
    for (N, I, O, G) in [(2048, 40, 100, 8), (2048, 21, 23, 20)]:
        d = wl.random_layer(N, I, O, G, dtype=dtype, base=True, seed=9)
        (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
        grid = (d["lo"], d["hi"], d["G"])
        xt, Ct, Wt, dyt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype), to_dev(dy, "f32")
        say("split %s %dx%dx%d G=%d" % (dtype, N, I, O, G))
        both = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
        only_c = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, need_dW=False, variant="mfma")
        only_w = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, need_dC=False, variant="mfma")
        again = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
        y = F.kan_forward(xt, Ct, Wt, grid, "mfma")
        y2 = F.kan_forward(xt, Ct, Wt, grid, "mfma")
        _sync()
        assert only_c[2] is None and only_w[1] is None
        assert torch.equal(both[1], only_c[1]) and torch.equal(both[2], only_w[2])
        assert torch.equal(both[1], again[1]) and torch.equal(both[2], again[2]) and torch.equal(y, y2)
        err, tol = metric(dtype)
        _, rdC, rdW = oracle.layer_backward(x, C, W, dy, *grid, need=("dC", "dW"))
        assert err(_np(both[1]), rdC) <= tol and err(_np(both[2]), rdW) <= tol
        assert err(_np(y), oracle.layer_forward(x, C, W, *grid)) <= tol


def test_tail_split(F):
    """Launches with a little over one round of output tiles: the tile rows
    that fill whole rounds run their whole k range and write their outputs,
    and only the last tile rows run in fixed k slices that fill the final
    round, summed in slice order.  The forward (4252 rows x 4066 outputs:
    17 x 16 tiles, of which the last tile row is sliced; both the 2:4 and
    the dense form) and dC (4302 outputs x 342 inputs, Kb = 12: 17 x 17
    tiles, the last 2 tile rows sliced) against the oracle in full, with
    ragged edges on every side, and bitwise the same on a second call."""
    import torch
    dtype = "bf16"
    err, tol = metric(dtype)
    d = wl.random_layer(4252, 128, 4066, 8, dtype=dtype, base=True, seed=31)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype)
    ry = oracle.layer_forward(x, C, W, *grid)
    for dense in (False, True):
        say("tail split forward 4252x128x4066 dense=%d" % dense)
        y = F.kan_forward(xt, Ct, Wt, grid, "mfma", dense_forward=dense)
        y2 = F.kan_forward(xt, Ct, Wt, grid, "mfma", dense_forward=dense)
        _sync()
        assert torch.equal(y, y2)
        assert err(_np(y), ry) <= tol
    d = wl.random_layer(1000, 342, 4302, 8, dtype=dtype, base=True, seed=32)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    xt, Ct, Wt, dyt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype), to_dev(dy, "f32")
    say("tail split dC 1000x342x4302")
    g1 = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
    g2 = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
    _sync()
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    _, rdC, rdW = oracle.layer_backward(x, C, W, dy, *grid, need=("dC", "dW"))
    assert err(_np(g1[1]), rdC) <= tol and err(_np(g1[2]), rdW) <= tol


def test_tail_split_dc_f32(F):
    """The float32 dC with the same tail split (17 x 17 tiles, the last 2
    tile rows of outputs in batch slices) against the oracle in full, and
    bitwise the same on a second call."""
    import torch
    dtype = "f32"
    err, tol = metric(dtype)
    d = wl.random_layer(1000, 342, 4302, 8, dtype=dtype, base=True, seed=34)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt, dyt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype), to_dev(dy, "f32")
    say("tail split dC f32 1000x342x4302")
    g1 = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
    g2 = F.kan_backward(xt, Ct, Wt, dyt, grid, need_dx=False, variant="mfma")
    _sync()
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    _, rdC, rdW = oracle.layer_backward(x, C, W, dy, *grid, need=("dC", "dW"))
    assert err(_np(g1[1]), rdC) <= tol and err(_np(g1[2]), rdW) <= tol


@pytest.mark.parametrize("shape", [(300, 40, 2000, 8, True), (700, 100, 1793, 3, False), (500, 60, 600, 5, True)])
def test_materialized_basis(F, shape):
    """bf16 layers with few columns per input (Kb = 12, 6 and 9) build their
    dense basis operands once in HBM, the forward's from 8 output tiles and
    dC's from 3 (the third shape: dC only): the forward (dense form) and dC
    against the oracle in full, and the forward bitwise equal to
    kan_forward_static, whose fixed workspace keeps the basis generated
    inside the contraction (the same LDS tiles, so the same bits)."""
    import torch
    N, I, O, G, base = shape
    dtype = "bf16"
    err, tol = metric(dtype)
    d = wl.random_layer(N, I, O, G, dtype=dtype, base=base, seed=33)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, dyt = to_dev(x, dtype), to_dev(C, dtype), to_dev(dy, "f32")
    Wt = to_dev(W, dtype) if base else None
    say("materialized basis %dx%dx%d G=%d base=%d" % shape)
    y = F.kan_forward(xt, Ct, Wt, grid, "mfma", dense_forward=True)
    ys = F.kan_forward_static(xt, Ct, Wt, grid, "mfma", dense_forward=True)
    g = F.kan_backward(xt, Ct, Wt, dyt, grid, variant="mfma")
    _sync()
    assert torch.equal(y, ys)
    assert err(_np(y), oracle.layer_forward(x, C, W, *grid)) <= tol
    rdx, rdC, rdW = oracle.layer_backward(x, C, W, dy, *grid)
    assert err(_np(g[0]), rdx) <= tol and err(_np(g[1]), rdC) <= tol
    if base:
        assert err(_np(g[2]), rdW) <= tol


@pytest.mark.parametrize("variant", ["mfma", "gather"])
def test_empty_batch(F, variant):
    import torch
    say("empty batch", variant)
    C = torch.randn(5, 7, 11, device="cuda:0")
    W = torch.randn(5, 7, device="cuda:0")
    x = torch.empty(0, 7, device="cuda:0")
    y = F.kan_forward(x, C, W, (-1.0, 1.0, 8), variant)
    dx, dC, dW = F.kan_backward(x, C, W, torch.empty(0, 5, device="cuda:0"), (-1.0, 1.0, 8),
                                variant=variant)
    _sync()
    assert y.shape == (0, 5) and dx.shape == (0, 7)
    assert torch.count_nonzero(dC) == 0 and torch.count_nonzero(dW) == 0


def test_binding_rejects_bad_outputs_and_workspaces(F):
    """The Python binding refuses, before any launch, an ``out`` tensor of the
    wrong shape and a workspace smaller than the bytes it declares (the
    library trusts the declared size), for the layer, the grouped activation
    and the 2-D layer."""
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    say("binding checks")
    dev = "cuda:0"
    grid = (-1.0, 1.0, 5)
    x = torch.rand(40, 6, device=dev) * 2 - 1
    C = torch.randn(3, 6, 8, device=dev)
    W = torch.randn(3, 6, device=dev)
    desc = F.layer_desc(x, C, W, grid, "mfma")
    n = F.kan_workspace_size(desc, L.KAN_PASS_FORWARD)
    assert n > 0
    with pytest.raises(ValueError, match="y must be"):
        F.kan_forward(x, C, W, grid, "mfma", out=torch.empty(40, 2, device=dev))
    with pytest.raises(ValueError, match="declared"):
        F.kan_forward(x, C, W, grid, "mfma", ws=(torch.empty(n - 1, dtype=torch.uint8, device=dev), n))
    nb = F.kan_workspace_size(desc, L.KAN_PASS_BACKWARD)
    with pytest.raises(ValueError, match="declared"):
        F.kan_backward(x, C, W, torch.randn(40, 3, device=dev), grid, variant="mfma",
                       ws=(torch.empty(nb // 2, dtype=torch.uint8, device=dev), nb))
    with pytest.raises(ValueError, match="device tensor"):
        F.kan_forward(x, C, W, grid, "mfma", ws=(torch.empty(n, dtype=torch.uint8), n))
    with pytest.raises(ValueError, match="dy must be"):
        F.kan_prepare(x, C, W, grid, L.KAN_PASS_BACKWARD, dy=torch.randn(40, 4, device=dev), variant="mfma")
    Cg = torch.randn(2, 8, device=dev)
    with pytest.raises(ValueError, match="y must be"):
        F.kan_group_forward(x, Cg, grid, out=torch.empty(40, 5, device=dev))
    gd = F.group_desc(x, Cg, grid)
    ng = F.kan_group_workspace_size(gd)
    with pytest.raises(ValueError, match="declared"):
        F.kan_group_backward(x, Cg, torch.randn(40, 6, device=dev), grid,
                             ws=(torch.empty(max(ng - 4, 1), dtype=torch.uint8, device=dev), ng))
    Cs = torch.randn(3, 3, 8, 8, device=dev)
    with pytest.raises(ValueError, match="y must be"):
        F.kan_surface_forward(x, Cs, grid, out=torch.empty(39, 3, device=dev))
    sd = F.surface_desc(x, Cs, grid)
    ns = F.kan_surface_workspace_size(sd, L.KAN_PASS_BACKWARD)
    with pytest.raises(ValueError, match="declared"):
        F.kan_surface_backward(x, Cs, torch.randn(40, 3, device=dev), grid,
                               ws=(torch.empty(max(ns - 256, 1), dtype=torch.uint8, device=dev), ns))
    # correct outputs and workspaces still work
    y = torch.empty(40, 3, device=dev)
    F.kan_forward(x, C, W, grid, "mfma", out=y, ws=(torch.empty(n, dtype=torch.uint8, device=dev), n))
    _sync()
    ref = oracle.layer_forward(_np(x).astype(np.float64), _np(C).astype(np.float64),
                               _np(W).astype(np.float64), -1.0, 1.0, 5)
    assert rel_inf(_np(y), ref) <= TOL_F32


@pytest.mark.parametrize("variant", ["mfma", "gather"])
def test_output_guards_and_nonfinite_inputs(F, variant):
    """Outputs written exactly in place (NaN canaries around them stay NaN);
    non-finite inputs neither crash nor disturb other rows."""
    import ctypes
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    say("guards", variant)
    N, I, O, G = 130, 21, 19, 8
    d = wl.random_layer(N, I, O, G, dtype="f32", base=True, seed=11)
    (C, W), x, dy = d["layers"][0], d["x"].copy(), d["dy"]
    bad_rows = [3, 77]
    x[3, 4], x[77, 0] = np.nan, np.inf
    dev = "cuda:0"
    xt, Ct, Wt, dyt = to_dev(x, "f32"), to_dev(C, "f32"), to_dev(W, "f32"), to_dev(dy, "f32")
    G4 = 64  # guard floats each side (keeps 16-byte alignment)

    def guarded(n):
        buf = torch.full((n + 2 * G4,), float("nan"), device=dev)
        return buf, buf[G4:G4 + n]

    yb, y = guarded(N * O)
    dxb, dx = guarded(N * I)
    dCb, dC = guarded(O * I * (G + 3))
    dWb, dW = guarded(O * I)
    desc = F.layer_desc(xt, Ct, Wt, (-1.0, 1.0, G), variant)
    wsf, nf = F.workspace(desc, 0, dev)
    wsb, nb = F.workspace(desc, 1, dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.check(L.lib().kan_forward(ctypes.byref(desc), p(xt), p(Ct), p(Wt), p(y), p(wsf), nf, s), "fwd")
    L.check(L.lib().kan_backward(ctypes.byref(desc), p(xt), p(Ct), p(Wt), p(dyt), p(dx), p(dC), p(dW),
                                 p(wsb), nb, s), "bwd")
    _sync()
    for buf in (yb, dxb, dCb, dWb):
        assert torch.isnan(buf[:G4]).all() and torch.isnan(buf[-G4:]).all()
    ok = np.setdiff1d(np.arange(N), bad_rows)
    ref_y = oracle.layer_forward(x[ok], C, W, -1.0, 1.0, G)
    assert rel_inf(_np(y).reshape(N, O)[ok], ref_y) <= TOL_F32
    ref_dx = oracle.layer_backward(x[ok], C, W, dy[ok], -1.0, 1.0, G, need=("dx",))[0]
    assert rel_inf(_np(dx).reshape(N, I)[ok], ref_dx) <= TOL_F32
    # the spline part of dC never sees the bad inputs: their basis is empty
    xc = x.copy()
    xc[3, 4] = xc[77, 0] = 1e6
    ref_dC = oracle.layer_backward(xc, C, W, dy, -1.0, 1.0, G, need=("dC",))[1]
    assert rel_inf(_np(dC).reshape(O, I, G + 3), ref_dC) <= TOL_F32


# ---------------------------------------------------------------------------
# the workloads
def run_net_gpu(F, d, variant="auto"):
    """Forward + backward of the whole chain through the C ABI."""
    import torch
    dt = d["dtype"]
    grid = (d["lo"], d["hi"], d["G"])
    xs = [to_dev(d["x"], dt)]
    Ls = [(to_dev(C, dt), to_dev(W, dt)) for C, W in d["layers"]]
    for li, (Ct, Wt) in enumerate(Ls):
        y = F.kan_forward(xs[-1], Ct, Wt, grid, variant)
        if li + 1 < len(Ls):
            y = F.kan_cast_f32_to_bf16(y) if dt == "bf16" else y
        xs.append(y)
    g = to_dev(d["dy"], "f32")
    grads = [None] * len(Ls)
    for li in range(len(Ls) - 1, -1, -1):
        Ct, Wt = Ls[li]
        dx, dC, dW = F.kan_backward(xs[li], Ct, Wt, g, grid, variant=variant)
        grads[li] = (dC, dW)
        g = dx
    torch.cuda.synchronize()
    return xs[-1], g, grads


# The oracle's full result for the last workload checked in full, shared by
# the variants that run it (the c3 G = 8 chain is ~0.57 TFLOP of float64).
_FULL = {}


def _full_oracle(d, k):
    key = (d["name"], d["G"], d["N"], k)
    if key not in _FULL:
        _FULL.clear()
        lo, hi, G = d["lo"], d["hi"], d["G"]
        acts = oracle.network_forward(d["x"], d["layers"], lo, hi, G, bf16_between=d["dtype"] == "bf16", k=k)
        dx0, grads = oracle.network_backward(acts, d["layers"], d["dy"], lo, hi, G, k=k)
        _FULL[key] = (acts[-1], dx0, grads)
    return _FULL[key]


def check_net(F, d, rows=None, pairs=None, variant="auto", seed=0):
    """A whole chain on the GPU against the oracle.  ``rows=None`` and
    ``pairs=None``: every entry of y, dx and each layer's dC / dW_base.
    Otherwise y and dx on ``rows`` seeded rows and dC / dW_base on ``pairs``
    seeded (j, i) pairs per layer, each a sum over every row."""
    name = d["name"]
    lo, hi, G = d["lo"], d["hi"], d["G"]
    layers = d["layers"]
    k = layers[0][0].shape[2] - G                  # spline degree
    bf = d["dtype"] == "bf16"
    err, tol = metric(d["dtype"])
    say("workload %s G=%d D=%d N=%d variant=%s: GPU" % (name, G, k, d["N"], variant))
    y, dx0, grads = run_net_gpu(F, d, variant)
    errs = {}
    if rows is None and pairs is None:
        say("workload %s: oracle in full" % name)
        ry, rdx, rgrads = _full_oracle(d, k)
        errs["y"] = err(_np(y), ry)
        errs["dx0"] = err(_np(dx0), rdx)
        for li, (C, W) in enumerate(layers):
            errs["dC%d" % li] = err(_np(grads[li][0]).reshape(C.shape), rgrads[li][0])
            if W is not None:
                errs["dW%d" % li] = err(_np(grads[li][1]), rgrads[li][1])
    else:
        assert k == 3, "sampled checks are written for the cubic layer"
        N = d["N"]
        R = np.arange(N) if rows is None else wl.sample_indices(N, rows, seed)
        say("workload %s: oracle rows=%d pairs=%d" % (name, len(R), pairs))
        acts = oracle.network_forward(d["x"][R], layers, lo, hi, G, bf16_between=bf)
        dxr, _ = oracle.network_backward(acts, layers, d["dy"][R], lo, hi, G)
        errs["y"] = err(_np(y)[R], acts[-1])
        errs["dx0"] = err(_np(dx0)[R], dxr)
        # per-layer coefficient gradients on sampled (j, i) pairs over all rows
        for li in range(len(layers)):
            C, W = layers[li]
            O, I = C.shape[0], C.shape[1]
            P = wl.sample_pairs(O, I, pairs, seed + li)
            xin = _layer_input_columns(d, li, np.unique(P[:, 1]))
            gin = _upstream_columns(d, li, np.unique(P[:, 0]))
            dCp = np.zeros((len(P), G + 3))
            dWp = np.zeros(len(P))
            for q, (j, i) in enumerate(P):
                c, w = oracle.coef_grad_pairs(xin[i][:, None], gin[j][:, None], [[0, 0]], lo, hi, G,
                                              W is not None)
                dCp[q] = c[0]
                if W is not None:
                    dWp[q] = w[0]
            gC = _np(grads[li][0]).reshape(O, I, G + 3)[P[:, 0], P[:, 1]]
            errs["dC%d" % li] = err(gC, dCp)
            if W is not None:
                errs["dW%d" % li] = err(_np(grads[li][1])[P[:, 0], P[:, 1]], dWp)
    say("workload %s errors: %s" % (name, " ".join("%s=%.2e" % kv for kv in errs.items())))
    for key, e in errs.items():
        assert e <= tol, "%s: %s error %.3e > %.0e" % (name, key, e, tol)


def _layer_input_columns(d, li, cols):
    """Columns of layer li's input over every row (layer 0: x; layer 1: the
    first layer's output columns, bf16-rounded for bf16 networks)."""
    if li == 0:
        return {int(i): d["x"][:, i].astype(np.float64) for i in cols}
    assert li == 1
    C0, W0 = d["layers"][0]
    lo, hi, G = d["lo"], d["hi"], d["G"]
    cols = np.asarray(cols)
    y = oracle.layer_forward(d["x"], C0[cols], None if W0 is None else W0[cols], lo, hi, G)
    if d["dtype"] == "bf16":
        y = oracle.round_bf16(y)
    return {int(c): y[:, k] for k, c in enumerate(cols)}


def _upstream_columns(d, li, cols):
    """Columns of the gradient arriving at layer li's output, over every row."""
    nl = len(d["layers"])
    if li == nl - 1:
        return {int(j): d["dy"][:, j].astype(np.float64) for j in cols}
    assert li == 0 and nl == 2
    # dy at layer 0's output = dx of layer 1; input column j of layer 1 needs
    # only x1[:, j], C1[:, j, :], W1[:, j]
    C1, W1 = d["layers"][1]
    lo, hi, G = d["lo"], d["hi"], d["G"]
    x1 = _layer_input_columns(d, 1, cols)
    out = {}
    for j in cols:
        j = int(j)
        dxj, _, _ = oracle.layer_backward(x1[j][:, None], C1[:, j:j + 1, :],
                                          None if W1 is None else W1[:, j:j + 1], d["dy"],
                                          lo, hi, G, need=("dx",))
        out[j] = dxj[:, 0]
    return out


# Parity at the sizes the workloads are defined at: c1, c2 and c3 at G = 8
# in full (every entry of every output); c3 at G = 20 and 50 on 512 seeded
# rows, c4 on 256 and c5 on 128, and 256 seeded (j, i) pairs of dC / dW_base
# per layer, each a sum over every row.  The grid sweep is the one of the
# InKAN page's "Performance" table, the chains its "Quick Start" network and
# the KAT channel mixer of the FlashKAT abstract.
@pytest.mark.parametrize("variant", ["auto", "mfma", "gather"])
def test_workload_c1(F, variant):
    check_net(F, wl.make_workload("c1"), variant=variant)


def check_layers(F, d, variant):
    """Each layer of a chain on its own, in full: a layer's input and its
    upstream gradient are the oracle's own intermediates rounded to the
    storage dtype, so only that layer's kernels are measured."""
    lo, hi, G = d["lo"], d["hi"], d["G"]
    layers = d["layers"]
    dt = d["dtype"]
    err, tol = metric(dt)
    acts = oracle.network_forward(d["x"], layers, lo, hi, G, bf16_between=dt == "bf16")
    ups = [None] * len(layers)
    g = d["dy"].astype(np.float64)
    for li in range(len(layers) - 1, -1, -1):
        ups[li] = g
        g = oracle.layer_backward(acts[li], *layers[li], g, lo, hi, G, need=("dx",))[0]
    for li, (C, W) in enumerate(layers):
        xl = acts[li].astype(np.float32)
        gl = ups[li].astype(np.float32)
        say("layer %d of %s on its own, variant=%s" % (li, d["name"], variant))
        one = dict(d, x=xl, dy=gl, layers=[(C, W)])
        got = _layer_on_gpu(F, one, variant)
        ref = _layer_oracle(one)
        errs = {k: err(a, r) for k, a, r in zip(("y", "dx", "dC", "dW"), got, ref) if r is not None}
        say("  errors: " + " ".join("%s=%.2e" % kv for kv in errs.items()))
        for k, e in errs.items():
            assert e <= tol, "layer %d %s error %.3e > %.0e" % (li, k, e, tol)


@pytest.mark.parametrize("variant", ["auto", "mfma", "gather"])
def test_workload_c2(F, variant):
    check_net(F, wl.make_workload("c2"), variant=variant)


# The c2 chain with splines of degree 2 and 5 (the FlashKAN page's degree-k
# basis): the float32 forward of a chain at any degree keeps the next
# layer's B' from pushing it past 1e-5.
@pytest.mark.parametrize("D", [2, 5])
@pytest.mark.parametrize("variant", ["auto", "mfma", "gather"])
def test_workload_c2_degree(F, D, variant):
    check_net(F, wl.make_workload("c2", degree=D), variant=variant)


@pytest.mark.parametrize("variant", ["mfma", "gather"])
def test_workload_c2_per_layer(F, variant):
    check_layers(F, wl.make_workload("c2"), variant)


@pytest.mark.parametrize("variant", ["auto", "mfma"])
def test_workload_c3_full(F, variant):
    check_net(F, wl.make_workload("c3", G=8), variant=variant)


@pytest.mark.parametrize("G", [20, 50])
@pytest.mark.parametrize("variant", ["auto", "mfma"])
def test_workload_c3(F, G, variant):
    check_net(F, wl.make_workload("c3", G=G), rows=512, pairs=256, variant=variant)


def test_workload_c4(F):
    check_net(F, wl.make_workload("c4"), rows=256, pairs=256)


def test_workload_c5(F):
    check_net(F, wl.make_workload("c5"), rows=128, pairs=256)
