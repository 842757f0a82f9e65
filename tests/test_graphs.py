"""GPU: the entry points under HIP graph capture and on concurrent streams.

A training step (forward, dx, dC) of the layer, the grouped activation and the
2-D layer is captured once into a HIP graph (through ``torch.cuda.graph``, on
its capture stream) with its workspaces allocated beforehand, then replayed
several times with eager work and synchronisations between the replays.
Every replay must equal the eager results bitwise: the library records no
memset nodes (zero fills are kernels) and allocates nothing.  The same steps
on two streams at once must also match their eager results (the library
keeps no mutable global state).
"""

import ctypes

import numpy as np
import pytest

import workloads as wl
from kan_testutil import ensure_built, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    ensure_built()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kolmogorov_arnold_network_amd import _lib as L
    from kolmogorov_arnold_network_amd import functional as F
    return torch, L, F


def _layer_step(torch, L, F):
    """Inputs, outputs and a step closure for a bf16 layer with a base branch
    (structured-sparse forward, k-split dC)."""
    d = wl.random_layer(300, 40, 24, 20, dtype="bf16", base=True, seed=31)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt = to_dev(x, "bf16"), to_dev(C, "bf16"), to_dev(W, "bf16")
    dyt = to_dev(dy, "f32")
    desc = F.layer_desc(xt, Ct, Wt, grid)
    wsf = F.workspace(desc, L.KAN_PASS_FORWARD, xt.device)
    wsb = F.workspace(desc, L.KAN_PASS_BACKWARD, xt.device)
    y = torch.empty(300, 24, device="cuda:0")
    dx = torch.empty(300, 40, device="cuda:0")
    dC = torch.empty(C.shape, device="cuda:0")
    dW = torch.empty(W.shape, device="cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = L.lib()

    def step():
        S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L.check(lib.kan_forward(ctypes.byref(desc), P(xt), P(Ct), P(Wt), P(y), P(wsf[0]), wsf[1], S), "fwd")
        L.check(lib.kan_backward(ctypes.byref(desc), P(xt), P(Ct), P(Wt), P(dyt), P(dx), P(dC), P(dW),
                                 P(wsb[0]), wsb[1], S), "bwd")
    return step, (y, dx, dC, dW)


def _layer_built_step(torch, L, F):
    """A bf16 layer with 12 columns per input and 2000 outputs (dense forward
    flag): both passes build their basis operands in the workspace
    (gen_pack_kernel) before the contractions load them."""
    d = wl.random_layer(300, 40, 2000, 8, dtype="bf16", base=True, seed=35)
    (C, W), x, dy = d["layers"][0], d["x"], d["dy"]
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, Wt = to_dev(x, "bf16"), to_dev(C, "bf16"), to_dev(W, "bf16")
    dyt = to_dev(dy, "f32")
    desc = F.layer_desc(xt, Ct, Wt, grid, "mfma", L.KAN_FLAG_DENSE_FORWARD)
    wsf = F.workspace(desc, L.KAN_PASS_FORWARD, xt.device)
    wsb = F.workspace(desc, L.KAN_PASS_BACKWARD, xt.device)
    y = torch.empty(300, 2000, device="cuda:0")
    dx = torch.empty(300, 40, device="cuda:0")
    dC = torch.empty(C.shape, device="cuda:0")
    dW = torch.empty(W.shape, device="cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = L.lib()

    def step():
        S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L.check(lib.kan_forward(ctypes.byref(desc), P(xt), P(Ct), P(Wt), P(y), P(wsf[0]), wsf[1], S), "fwd")
        L.check(lib.kan_backward(ctypes.byref(desc), P(xt), P(Ct), P(Wt), P(dyt), P(dx), P(dC), P(dW),
                                 P(wsb[0]), wsb[1], S), "bwd")
    return step, (y, dx, dC, dW)


def _grouped_step(torch, L, F):
    d = wl.random_grouped(500, 300, 7, 8, dtype="bf16", seed=32)
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, dyt = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16"), to_dev(d["dy"], "f32")
    desc = F.group_desc(xt, Ct, grid)
    n = F.kan_group_workspace_size(desc)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty(500, 300, device="cuda:0")
    dx = torch.empty(500, 300, device="cuda:0")
    dC = torch.empty(7, 11, device="cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = L.lib()

    def step():
        S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L.check(lib.kan_group_forward(ctypes.byref(desc), P(xt), P(Ct), P(y), S), "fwd")
        L.check(lib.kan_group_backward(ctypes.byref(desc), P(xt), P(Ct), P(dyt), P(dx), P(dC), P(ws), n, S),
                "bwd")
    return step, (y, dx, dC)


def _surface_step(torch, L, F):
    d = wl.random_surface(260, 6, 20, 7, dtype="bf16", seed=33)
    grid = (d["lo"], d["hi"], d["G"])
    xt, Ct, dyt = to_dev(d["x"], "bf16"), to_dev(d["C"], "bf16"), to_dev(d["dy"], "f32")
    desc = F.surface_desc(xt, Ct, grid)
    nf = F.kan_surface_workspace_size(desc, L.KAN_PASS_FORWARD)
    nb = F.kan_surface_workspace_size(desc, L.KAN_PASS_BACKWARD)
    wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda:0")
    wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    y = torch.empty(260, 20, device="cuda:0")
    dx = torch.empty(260, 12, device="cuda:0")
    dC = torch.empty(Ct.shape, device="cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = L.lib()

    def step():
        S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L.check(lib.kan_surface_forward(ctypes.byref(desc), P(xt), P(Ct), P(y), P(wsf), nf, S), "fwd")
        L.check(lib.kan_surface_backward(ctypes.byref(desc), P(xt), P(Ct), P(dyt), P(dx), P(dC), P(wsb), nb, S),
                "bwd")
    return step, (y, dx, dC)


STEPS = {"layer": _layer_step, "layer_built": _layer_built_step, "grouped": _grouped_step,
         "surface": _surface_step}


@pytest.mark.parametrize("name", sorted(STEPS))
def test_graph_replays_match_eager(env, name):
    torch, L, F = env
    step, outs = STEPS[name](torch, L, F)
    step()
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # warm-up on the side stream (function attributes set)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        o.fill_(12345.0)
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(-7.0)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(o.cpu().numpy(), e), (name, rep)


def test_two_streams_at_once(env):
    torch, L, F = env
    step_a, outs_a = _layer_step(torch, L, F)
    step_b, outs_b = _surface_step(torch, L, F)
    step_a()
    step_b()
    torch.cuda.synchronize()
    ea = [o.cpu().numpy().copy() for o in outs_a]
    eb = [o.cpu().numpy().copy() for o in outs_b]
    for o in outs_a + outs_b:
        o.fill_(0.5)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(sa):
            step_a()
        with torch.cuda.stream(sb):
            step_b()
    torch.cuda.synchronize()
    for o, e in zip(outs_a, ea):
        assert np.array_equal(o.cpu().numpy(), e)
    for o, e in zip(outs_b, eb):
        assert np.array_equal(o.cpu().numpy(), e)
