"""kan_forward_static, the forward that takes its workspace from the library's
static device array, against kan_forward on the same inputs.

Both run the same kernels, so the outputs must be bitwise equal; each is also
held to the layer's tolerance against the float64 oracle.  Each case makes
two calls in a row, the second on a smaller layer, so the second call runs
on an array that still holds the first call's contents.
"""

import ctypes
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from kan_testutil import ensure_built, metric, to_dev

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


def _static_forward(L, desc, x, C, W, y):
    """One kan_forward_static call through the C ABI on the current stream."""
    import torch
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return L.lib().kan_forward_static(ctypes.byref(desc), p(x), p(C), p(W), p(y), s)


# (N, I, O, G, base, dtype, variant): a larger layer, then a smaller one.
# float32 AUTO: the gather forward with its inputs split (float64 partials
# in the array); mfma: packed C' and the slices' partial outputs in the
# array; bf16: the structured-sparse forward's packed operand.
PAIRS = [
    [(1024, 784, 64, 8, True, "f32", "auto"), (300, 100, 50, 8, True, "f32", "auto")],
    [(1024, 784, 64, 8, True, "f32", "mfma"), (257, 61, 33, 5, False, "f32", "mfma")],
    [(2000, 300, 200, 20, True, "bf16", "mfma"), (500, 40, 30, 20, True, "bf16", "mfma")],
    [(1024, 64, 10, 8, True, "f32", "gather"), (70, 250, 66, 8, False, "f32", "gather")],
]


@pytest.mark.parametrize("pair", PAIRS, ids=["-".join(str(v) for v in p[0]) for p in PAIRS])
def test_static_forward_matches_kan_forward(F, pair):
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    for k, (N, I, O, G, base, dtype, variant) in enumerate(pair):
        say("static forward call %d: %dx(%d->%d) G=%d base=%s %s %s" % (k, N, I, O, G, base, dtype, variant))
        d = wl.random_layer(N, I, O, G, dtype=dtype, base=base, seed=31 + k)
        (C, W), x = d["layers"][0], d["x"]
        grid = (d["lo"], d["hi"], G)
        xt, Ct, Wt = to_dev(x, dtype), to_dev(C, dtype), to_dev(W, dtype)
        desc = F.layer_desc(xt, Ct, Wt, grid, variant)
        assert 0 <= F.kan_workspace_size(desc, L.KAN_PASS_FORWARD) <= L.KAN_STATIC_SCRATCH_BYTES
        y_ref = F.kan_forward(xt, Ct, Wt, grid, variant)
        y = torch.full((N, O), float("nan"), dtype=torch.float32, device="cuda:0")
        L.check(_static_forward(L, desc, xt, Ct, Wt, y), "kan_forward_static")
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "static forward differs from kan_forward"
        err, tol = metric(dtype)
        e = err(y.cpu().numpy(), oracle.layer_forward(x, C, W, *grid))
        say("  error vs oracle %.2e" % e)
        assert e <= tol


def test_static_forward_functional_and_rejection(F):
    """The binding's kan_forward_static gives the same bits; a layer whose
    forward workspace exceeds the array is refused before any work, and the
    output is left untouched."""
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    d = wl.random_layer(129, 37, 19, 8, dtype="f32", base=True, seed=41)
    (C, W), x = d["layers"][0], d["x"]
    grid = (d["lo"], d["hi"], 8)
    xt, Ct, Wt = to_dev(x, "f32"), to_dev(C, "f32"), to_dev(W, "f32")
    for variant in ("auto", "mfma", "gather"):
        y = F.kan_forward_static(xt, Ct, Wt, grid, variant)
        y_ref = F.kan_forward(xt, Ct, Wt, grid, variant)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
    # 65536 x 4096 -> 4096 at G = 20, bf16: 0.8 GB of packed operand
    big = L.make_desc(65536, 4096, 4096, -1.0, 1.0, 20, L.KAN_BF16, True, L.KAN_VARIANT_AUTO, 0)
    small = torch.full((4, 4), 7.0, device="cuda:0")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = L.lib().kan_forward_static(ctypes.byref(big), p(xt), p(Ct), p(Wt), p(small), s)
    assert st == L.KAN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(small == 7.0)
