"""GPU parity of the 2-D tensor-product spline layer (``kan_surface_forward``
/ ``kan_surface_backward`` through the C ABI) against the float64 oracle
``oracle.surface``.

Tolerances as for the layer: float32 storage, normwise max relative error
<= 1e-5 per output; bf16 storage, relative Frobenius error <= 1e-2 (the
products of the basis values and dy are rounded to bf16 on the matrix
cores).  Small shapes are compared in full; they cover every operand
variant (pairs per k-tile, pairs per dC tile, pairs cut by dx tile edges,
one pair per whole tile).  The full-size workload s1 runs in the launch
configuration the benchmark times and is compared on seeded rows (y, dx) and
seeded (output, pair) blocks of dC, which the oracle sums over all rows.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from kan_testutil import ensure_built, metric, rel_fro, to_dev

pytestmark = pytest.mark.gpu


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


def _np(t):
    import torch
    torch.cuda.synchronize()
    return None if t is None else t.detach().float().cpu().numpy()


SMALL = [
    # N, P, O, G, dtype                  what it covers
    (37, 3, 5, 5, "f32"),               # Kb = 64: one pair per bf16 k-tile, two per fp32 tile edge
    (300, 7, 33, 8, "bf16"),            # Kb = 121: pairs cut by dx tile edges
    (64, 16, 40, 1, "f32"),             # Kb = 16: several pairs per k-tile and per dC tile
    (50, 5, 7, 1, "bf16"),              # Kb = 16 in bf16
    (129, 9, 17, 2, "bf16"),            # Kb = 25
    (77, 4, 300, 13, "f32"),            # Kb = 256: one pair per whole tile, O > 256
    (260, 6, 20, 7, "bf16"),            # Kb = 100
    (33, 40, 9, 5, "f32"),              # 40 pairs, 10 dx tiles
    (1, 1, 1, 3, "bf16"),               # smallest
    (200, 6, 600, 5, "bf16"),           # O > 512 in bf16: dC on the pair basis built once (Kb = 64)
    (64, 16, 700, 1, "bf16"),           # the same with Kb = 16
]


@pytest.mark.parametrize("N,P,O,G,dtype", SMALL)
def test_small(F, N, P, O, G, dtype):
    say("surface N=%d P=%d O=%d G=%d %s" % (N, P, O, G, dtype))
    d = wl.random_surface(N, P, O, G, dtype, seed=N + P)
    grid = (d["lo"], d["hi"], G)
    x, C, dy = to_dev(d["x"], dtype), to_dev(d["C"], dtype), to_dev(d["dy"], "f32")
    y = F.kan_surface_forward(x, C, grid)
    dx, dC = F.kan_surface_backward(x, C, dy, grid)
    ry = oracle.surface_forward(d["x"], d["C"], *grid)
    rdx, rdC = oracle.surface_backward(d["x"], d["C"], d["dy"], *grid)
    err, tol = metric(dtype)
    assert err(_np(y), ry) <= tol
    assert err(_np(dx), rdx) <= tol
    assert err(_np(dC), rdC) <= tol


def test_partial_outputs_determinism_and_empty(F):
    import torch
    d = wl.random_surface(500, 10, 70, 5, "bf16", seed=9)
    grid = (d["lo"], d["hi"], 5)
    x, C, dy = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16"), to_dev(d["dy"], "f32")
    dx, dC = F.kan_surface_backward(x, C, dy, grid)
    dx2, dC2 = F.kan_surface_backward(x, C, dy, grid)
    dxo, n1 = F.kan_surface_backward(x, C, dy, grid, need_dC=False)
    n2, dCo = F.kan_surface_backward(x, C, dy, grid, need_dx=False)
    assert n1 is None and n2 is None
    for a, b in ((dx, dx2), (dC, dC2), (dx, dxo), (dC, dCo)):
        assert np.array_equal(_np(a), _np(b))
    y1, y2 = F.kan_surface_forward(x, C, grid), F.kan_surface_forward(x, C, grid)
    assert np.array_equal(_np(y1), _np(y2))
    # empty batch: y and dx are empty, dC is zero
    xe = torch.empty(0, 20, dtype=torch.bfloat16, device="cuda:0")
    dye = torch.empty(0, 70, device="cuda:0")
    ye = F.kan_surface_forward(xe, C, grid)
    dxe, dCe = F.kan_surface_backward(xe, C, dye, grid)
    assert ye.shape == (0, 70) and dxe.shape == (0, 20)
    assert np.array_equal(_np(dCe), np.zeros(C.shape, np.float32))


def test_workload_s1(F):
    d = wl.make_surface("s1")
    N, P, O, G, lo, hi = d["N"], d["P"], d["O"], d["G"], d["lo"], d["hi"]
    say("surface workload s1: N=%d P=%d O=%d G=%d" % (N, P, O, G))
    grid = (lo, hi, G)
    x, C, dy = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16"), to_dev(d["dy"], "f32")
    y = F.kan_surface_forward(x, C, grid)
    dx, dC = F.kan_surface_backward(x, C, dy, grid)
    yn, dxn, dCn = _np(y), _np(dx), _np(dC)
    rows = wl.sample_indices(N, 64, seed=21)
    ry = oracle.surface_forward_rows(d["x"], d["C"], lo, hi, G, rows)
    rdx, _ = oracle.surface_backward(d["x"][rows], d["C"], d["dy"][rows], lo, hi, G)
    assert rel_fro(yn[rows], ry) <= 1e-2
    assert rel_fro(dxn[rows], rdx) <= 1e-2
    pairs = wl.sample_pairs(O, P, 24, seed=22)
    rdC = oracle.surface_coef_grad_pairs(d["x"], d["dy"], lo, hi, G, [tuple(q) for q in pairs])
    assert rel_fro(dCn[pairs[:, 0], pairs[:, 1]], rdC) <= 1e-2


@pytest.mark.parametrize("N,P,O", [(300, 7, 40), (1000, 3, 300), (64, 1, 1)])
def test_sparse_forward(F, N, P, O):
    """bf16, G = 5: the 2:4 structured-sparse forward (the default) against the
    dense form and the oracle; x includes knots and far-outside points."""
    d = wl.random_surface(N, P, O, 5, "bf16", seed=N + 7)
    grid = (d["lo"], d["hi"], 5)
    x, C = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16")
    ys = _np(F.kan_surface_forward(x, C, grid))
    yd = _np(F.kan_surface_forward(x, C, grid, dense_forward=True))
    ref = oracle.surface_forward(d["x"], d["C"], *grid)
    assert rel_fro(ys, ref) <= 1e-2
    assert rel_fro(yd, ref) <= 1e-2
    # same bf16 products in a different summation order
    assert rel_fro(ys, yd) <= 1e-5
