"""GPU parity of the grouped spline activation (``kan_group_forward`` /
``kan_group_backward`` through the C ABI) against the float64 oracle
``oracle.grouped``.

x, C and dy are exact in float32 (bf16 inputs hold bf16 values) and the
kernels compute in float32, so every case, bf16 storage included, is held to
the float32 bar: normwise max relative error <= 1e-5 per output tensor.

Small shapes are compared in full.  The full-size workloads (g1, g2) run in
the launch configuration the benchmark times and are compared on:

- y and dx on seeded rows (a row depends only on the same row of x and dy);
- dC exactly, for a dy that is zero outside seeded rows (same shapes, so the
  same grid, chunks and reduction order);
- dC for the full dy through two identities of the cubic B-splines that hold
  for every x in [lo, hi]: partition of unity, sum_m B_m(x) = 1, and linear
  precision, sum_m xi_m B_m(x) = x with the Greville abscissae
  xi_m = (t_{m+1} + t_{m+2} + t_{m+3}) / 3 = lo + (m - 1) h.  Summed against dy
  over a group's elements they give sum_m dC[g, m] = sum dy and
  sum_m xi_m dC[g, m] = sum dy * x, over all N * I / groups terms.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from kan_testutil import TOL_F32, ensure_built, rel_inf, to_dev

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


def _run(F, d):
    x, C, dy = to_dev(d["x"], d["dtype"]), to_dev(d["C"], d["dtype"]), to_dev(d["dy"], "f32")
    grid = (d["lo"], d["hi"], d["G"])
    y = F.kan_group_forward(x, C, grid)
    dx, dC = F.kan_group_backward(x, C, dy, grid)
    return _np(y), _np(dx), _np(dC)


SMALL = [
    # N, I, groups, G, dtype
    (37, 300, 7, 8, "f32"),        # I not a multiple of 256, ragged groups
    (64, 256, 256, 5, "f32"),      # one spline per channel, one channel block
    (5, 1000, 1, 20, "f32"),       # one group over four channel blocks
    (130, 77, 77, 50, "bf16"),     # per-channel, G = 50
    (300, 513, 3, 8, "bf16"),      # several row chunks per channel block
    (1, 1, 1, 1, "f32"),           # smallest
    (2000, 300, 300, 125, "f32"),  # largest G, coefficients read from memory
    (777, 600, 8, 125, "bf16"),    # largest G, coefficients staged in LDS
    (500, 300, 300, 29, "bf16"),   # the most coefficient rows that are staged
]


@pytest.mark.parametrize("N,I,groups,G,dtype", SMALL)
def test_small(F, N, I, groups, G, dtype):
    say("grouped N=%d I=%d groups=%d G=%d %s" % (N, I, groups, G, dtype))
    d = wl.random_grouped(N, I, groups, G, dtype, seed=N + I)
    y, dx, dC = _run(F, d)
    x64, C64, dy64 = (d[k].astype(np.float64) for k in ("x", "C", "dy"))
    ry = oracle.grouped_forward(x64, C64, d["lo"], d["hi"], G)
    rdx, rdC = oracle.grouped_backward(x64, C64, dy64, d["lo"], d["hi"], G)
    assert rel_inf(y, ry) <= TOL_F32
    assert rel_inf(dx, rdx) <= TOL_F32
    assert rel_inf(dC, rdC) <= TOL_F32


def test_partial_outputs_and_determinism(F):
    d = wl.random_grouped(1000, 700, 9, 8, "bf16", seed=5)
    x, C, dy = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16"), to_dev(d["dy"], "f32")
    grid = (d["lo"], d["hi"], d["G"])
    dx, dC = F.kan_group_backward(x, C, dy, grid)
    dx2, dC2 = F.kan_group_backward(x, C, dy, grid)
    dxo, none1 = F.kan_group_backward(x, C, dy, grid, need_dC=False)
    none2, dCo = F.kan_group_backward(x, C, dy, grid, need_dx=False)
    assert none1 is None and none2 is None
    for a, b in ((dx, dx2), (dC, dC2), (dx, dxo), (dC, dCo)):
        assert np.array_equal(_np(a), _np(b))
    y1, y2 = F.kan_group_forward(x, C, grid), F.kan_group_forward(x, C, grid)
    assert np.array_equal(_np(y1), _np(y2))


def test_empty_batch(F):
    import torch
    C = torch.randn(4, 11, device="cuda:0")
    x = torch.empty(0, 12, device="cuda:0")
    dy = torch.empty(0, 12, device="cuda:0")
    y = F.kan_group_forward(x, C, (-1.0, 1.0, 8))
    dx, dC = F.kan_group_backward(x, C, dy, (-1.0, 1.0, 8))
    assert y.shape == (0, 12) and dx.shape == (0, 12)
    assert np.array_equal(_np(dC), np.zeros((4, 11), np.float32))


def test_outputs_untouched_beyond_their_size(F):
    """y, dx and dC are written exactly where they are: guard words around
    them keep their pattern."""
    import torch
    d = wl.random_grouped(300, 301, 6, 8, "f32", seed=3)
    N, I, groups, K = 300, 301, 6, 11
    x, C, dy = to_dev(d["x"], "f32"), to_dev(d["C"], "f32"), to_dev(d["dy"], "f32")
    grid = (d["lo"], d["hi"], d["G"])
    pad = 64
    ybuf = torch.full((N * I + 2 * pad,), 7.5, device="cuda:0")
    y = ybuf[pad:pad + N * I].view(N, I)
    F.kan_group_forward(x, C, grid, out=y)
    yb = _np(ybuf)
    assert np.all(yb[:pad] == 7.5) and np.all(yb[-pad:] == 7.5)
    ry = oracle.grouped_forward(d["x"].astype(np.float64), d["C"].astype(np.float64), -1.0, 1.0, 8)
    assert rel_inf(yb[pad:-pad].reshape(N, I), ry) <= TOL_F32
    # dx / dC through the ABI with guarded buffers
    from kolmogorov_arnold_network_amd import _lib as L
    import ctypes
    desc = F.group_desc(x, C, grid)
    n = F.kan_group_workspace_size(desc)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dxb = torch.full((N * I + 2 * pad,), -3.25, device="cuda:0")
    dCb = torch.full((groups * K + 2 * pad,), -3.25, device="cuda:0")
    st = L.lib().kan_group_backward(ctypes.byref(desc), ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(C.data_ptr()), ctypes.c_void_p(dy.data_ptr()),
                                    ctypes.c_void_p(dxb.data_ptr() + pad * 4),
                                    ctypes.c_void_p(dCb.data_ptr() + pad * 4),
                                    ctypes.c_void_p(ws.data_ptr()), n,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    a, b = _np(dxb), _np(dCb)
    for buf in (a, b):
        assert np.all(buf[:pad] == -3.25) and np.all(buf[-pad:] == -3.25)


# ---------------------------------------------------------------------------
# full-size workloads
def _greville(lo, hi, G):
    h = (hi - lo) / G
    return lo + (np.arange(G + 3) - 1.0) * h


@pytest.mark.parametrize("name", ["g1", "g2"])
def test_workload(F, name):
    import torch
    d = wl.make_grouped(name)
    N, I, groups, G, lo, hi = d["N"], d["I"], d["groups"], d["G"], d["lo"], d["hi"]
    say("grouped workload %s: N=%d I=%d groups=%d G=%d" % (name, N, I, groups, G))
    assert d["x"].min() >= lo and d["x"].max() <= hi       # the identities need x in [lo, hi]
    x, C, dy = to_dev(d["x"], d["dtype"]), to_dev(d["C"], d["dtype"]), to_dev(d["dy"], "f32")
    grid = (lo, hi, G)
    y = F.kan_group_forward(x, C, grid)
    dx, dC = F.kan_group_backward(x, C, dy, grid)
    rows = wl.sample_indices(N, 96, seed={"g1": 1, "g2": 2}[name])
    x64, C64, dy64 = d["x"][rows].astype(np.float64), d["C"].astype(np.float64), d["dy"][rows].astype(np.float64)
    ry = oracle.grouped_forward(x64, C64, lo, hi, G)
    rdx, rdC_rows = oracle.grouped_backward(x64, C64, dy64, lo, hi, G)
    yn, dxn, dCn = _np(y), _np(dx), _np(dC)
    assert rel_inf(yn[rows], ry) <= TOL_F32
    assert rel_inf(dxn[rows], rdx) <= TOL_F32
    # dC for a dy restricted to the sampled rows
    mask = torch.zeros(N, 1, device="cuda:0")
    mask[torch.from_numpy(rows).to("cuda:0")] = 1.0
    _, dC_rows = F.kan_group_backward(x, C, dy * mask, grid, need_dx=False)
    assert rel_inf(_np(dC_rows), rdC_rows) <= TOL_F32
    # dC for the full dy: sums over every element of each group
    g = oracle.group_of(I, groups)
    dy_all = d["dy"].astype(np.float64)
    s0 = np.zeros(groups)
    s1 = np.zeros(groups)
    for r0 in range(0, N, 4096):
        blk = dy_all[r0:r0 + 4096]
        np.add.at(s0, g, blk.sum(axis=0))
        np.add.at(s1, g, (blk * d["x"][r0:r0 + 4096].astype(np.float64)).sum(axis=0))
    got0 = dCn.astype(np.float64).sum(axis=1)
    got1 = dCn.astype(np.float64) @ _greville(lo, hi, G)
    assert rel_inf(got0, s0) <= TOL_F32
    assert rel_inf(got1, s1) <= TOL_F32
