"""GPU: shapes whose tensors hold more than 2^31 elements, so that every index
computed in 32 bits would wrap.

A bf16 layer of 600,000 rows, 4096 -> 4096 (x, dy, y and dx each 2.46e9
elements), and a grouped activation of the same x.  Inputs are drawn on the
device from a seeded torch generator; the oracle checks seeded rows of y and
dx and seeded (output, input) pairs of dC, copying only those rows and
columns back to the host.  Tolerances are the layer's (bf16: relative
Frobenius 1e-2) and the grouped activation's (float32 arithmetic: 1e-5); the
grouped dC is checked exactly for a dy zeroed outside the seeded rows.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from kan_testutil import ensure_built, rel_fro, rel_inf

pytestmark = pytest.mark.gpu

N, I, O, G = 600_000, 4096, 4096, 5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    ensure_built()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kolmogorov_arnold_network_amd import functional as F
    g = torch.Generator(device="cuda:0").manual_seed(20261203)
    x = (torch.rand(N, I, device="cuda:0", generator=g) * 2.4 - 1.2).to(torch.bfloat16)
    assert x.numel() > 2 ** 31
    return torch, F, g, x


def test_layer_beyond_2_31_elements(env):
    torch, F, g, x = env
    say("layer %d x (%d -> %d), G=%d, bf16" % (N, I, O, G))
    C = (torch.randn(O, I, G + 3, device="cuda:0", generator=g) * 0.02).to(torch.bfloat16)
    W = (torch.randn(O, I, device="cuda:0", generator=g) / 64.0).to(torch.bfloat16)
    dy = torch.randn(N, O, device="cuda:0", generator=g)
    grid = (-1.0, 1.0, G)
    y = F.kan_forward(x, C, W, grid)
    dx, dC, dW = F.kan_backward(x, C, W, dy, grid)
    torch.cuda.synchronize()
    # seeded rows and the last one, whose elements sit past 2^31
    rows = torch.from_numpy(np.unique(np.append(wl.sample_indices(N, 12, seed=31), N - 1)))
    xs = x[rows.cuda()].float().cpu().numpy()
    Cn, Wn = C.float().cpu().numpy(), W.float().cpu().numpy()
    dys = dy[rows.cuda()].cpu().numpy()
    assert rel_fro(y[rows.cuda()].cpu().numpy(), oracle.layer_forward(xs, Cn, Wn, *grid)) <= 1e-2
    assert rel_fro(dx[rows.cuda()].cpu().numpy(), oracle.layer_backward_rows(xs, Cn, Wn, dys, *grid,
                                                                             np.arange(len(rows)))) <= 1e-2
    del y, dx
    pairs = wl.sample_pairs(O, I, 6, seed=32)
    pairs[-1] = (O - 1, I - 1)
    xcols = x[:, torch.from_numpy(pairs[:, 1]).cuda()].float().cpu().numpy()   # [N, 6]
    dycols = dy[:, torch.from_numpy(pairs[:, 0]).cuda()].cpu().numpy()
    local = np.stack([np.arange(6), np.arange(6)], axis=1)
    rdC, rdW = oracle.coef_grad_pairs(xcols, dycols, local, *grid, True)
    got_dC = dC[torch.from_numpy(pairs[:, 0]).cuda(), torch.from_numpy(pairs[:, 1]).cuda()].cpu().numpy()
    got_dW = dW[torch.from_numpy(pairs[:, 0]).cuda(), torch.from_numpy(pairs[:, 1]).cuda()].cpu().numpy()
    assert rel_fro(got_dC, rdC) <= 1e-2
    assert rel_fro(got_dW, rdW) <= 1e-2


def test_grouped_beyond_2_31_elements(env):
    torch, F, g, x = env
    groups = 16
    say("grouped activation %d x %d, %d groups, G=%d, bf16" % (N, I, groups, G))
    C = (torch.randn(groups, G + 3, device="cuda:0", generator=g) * 0.3).to(torch.bfloat16)
    dy = torch.randn(N, I, device="cuda:0", generator=g)
    grid = (-1.0, 1.0, G)
    y = F.kan_group_forward(x, C, grid)
    dx, dC = F.kan_group_backward(x, C, dy, grid)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.unique(np.append(wl.sample_indices(N, 8, seed=33), N - 1)))
    xs = x[rows.cuda()].float().cpu().numpy()
    Cn = C.float().cpu().numpy()
    dys = dy[rows.cuda()].cpu().numpy()
    assert rel_inf(y[rows.cuda()].cpu().numpy(), oracle.grouped_forward(xs, Cn, *grid)) <= 1e-5
    rdx, _ = oracle.grouped_backward(xs, Cn, dys, *grid)
    assert rel_inf(dx[rows.cuda()].cpu().numpy(), rdx) <= 1e-5
    del y, dx
    # dC exactly, for a dy zeroed outside the seeded rows (same shapes, so the
    # same chunks and reduction order; the last row's terms sit past 2^31)
    mask = torch.zeros(N, 1, device="cuda:0")
    mask[rows.cuda()] = 1.0
    dym = dy * mask
    del dy
    _, dCm = F.kan_group_backward(x, C, dym, grid, need_dx=False)
    _, rdC = oracle.grouped_backward(xs, Cn, dys, *grid)
    assert rel_inf(dCm.cpu().numpy(), rdC) <= 1e-5
