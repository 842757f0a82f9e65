"""``KANLayer`` / ``KANNetwork`` / ``KANGroupedActivation`` / ``KANSurfaceLayer``:
torch modules over the HIP library.

"KANLayer(in, out) replaces nn.Linear(in, out). Same interface, same
optimizer, same training loop" (InKAN project page, "Why InKAN?"): the layer
takes ``[..., in_features]`` and returns ``[..., out_features]``, and its
parameters are plain tensors that any torch optimizer updates.  Autograd
calls ``kan_backward``; torch only accumulates the returned gradients.
"""

import math

import torch

from . import functional as F


class KANFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, C, W, lo, hi, G, variant):
        ctx.grid = (lo, hi, G)
        ctx.variant = variant
        ctx.has_base = W is not None
        ctx.save_for_backward(x, C, W)
        return F.kan_forward(x, C, W, (lo, hi, G), variant)

    @staticmethod
    def backward(ctx, dy):
        x, C, W = ctx.saved_tensors
        need_x, need_C, need_W = ctx.needs_input_grad[:3]
        dx, dC, dW = F.kan_backward(x, C, W, dy.contiguous().float(), ctx.grid, need_dx=need_x,
                                    need_dC=need_C, need_dW=need_W and ctx.has_base,
                                    variant=ctx.variant)
        if dx is not None and dx.dtype != x.dtype:
            dx = dx.to(x.dtype)
        if dC is not None and dC.dtype != C.dtype:
            dC = dC.to(C.dtype)
        if dW is not None and dW.dtype != W.dtype:
            dW = dW.to(W.dtype)
        return dx, dC, dW, None, None, None, None


class CastBF16(torch.autograd.Function):
    """float32 -> bfloat16 on the device; the gradient passes through as float32."""

    @staticmethod
    def forward(ctx, t):
        return F.kan_cast_f32_to_bf16(t.contiguous())

    @staticmethod
    def backward(ctx, g):
        return g.float()


class KANLayer(torch.nn.Module):
    """One KAN layer: ``y_j = sum_i phi_ji(x_i)`` with cubic B-spline ``phi_ji``.

    Parameters: ``coef [out, in, grid_size + degree]`` and, with ``base=True``,
    ``base_weight [out, in]`` for the ``W_base * silu(x)`` branch.  ``dtype``
    (float32 or bfloat16) is the storage of inputs and parameters; outputs
    and gradients are computed in float32.  ``degree`` (1 .. 5) is the spline
    degree, 3 (cubic) by default.
    """

    def __init__(self, in_features, out_features, grid_size=8, grid_range=(-1.0, 1.0), base=True,
                 dtype=torch.float32, device=None, variant="auto", coef_std=0.1, degree=3):
        super().__init__()
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.grid_size = int(grid_size)
        self.grid_range = (float(grid_range[0]), float(grid_range[1]))
        self.variant = variant
        self.degree = int(degree)
        fk = dict(dtype=dtype, device=device)
        self.coef = torch.nn.Parameter(
            torch.randn(out_features, in_features, grid_size + self.degree, **fk) * coef_std)
        if base:
            self.base_weight = torch.nn.Parameter(
                torch.randn(out_features, in_features, **fk) / math.sqrt(in_features))
        else:
            self.register_parameter("base_weight", None)

    @property
    def grid(self):
        return (self.grid_range[0], self.grid_range[1], self.grid_size)

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if x2.dtype != self.coef.dtype:
            x2 = CastBF16.apply(x2) if self.coef.dtype == torch.bfloat16 else x2.to(self.coef.dtype)
        x2 = x2.contiguous()
        y = KANFunction.apply(x2, self.coef, self.base_weight, self.grid_range[0],
                              self.grid_range[1], self.grid_size, self.variant)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return "in=%d, out=%d, grid_size=%d, degree=%d, range=%s, base=%s, dtype=%s" % (
            self.in_features, self.out_features, self.grid_size, self.degree, self.grid_range,
            self.base_weight is not None, self.coef.dtype)


class KANNetwork(torch.nn.Module):
    """A chain of ``KANLayer`` with nothing in between (InKAN "Quick Start")."""

    def __init__(self, widths, **kw):
        super().__init__()
        self.layers = torch.nn.ModuleList(
            KANLayer(widths[l], widths[l + 1], **kw) for l in range(len(widths) - 1))

    def forward(self, x):
        for layer in self.layers:
            x = layer(x)
        return x


def _to_storage(x, dtype):
    if x.dtype == dtype:
        return x
    return CastBF16.apply(x) if dtype == torch.bfloat16 else x.to(dtype)


class GroupedFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, C, lo, hi, G):
        ctx.grid = (lo, hi, G)
        ctx.save_for_backward(x, C)
        return F.kan_group_forward(x, C, (lo, hi, G))

    @staticmethod
    def backward(ctx, dy):
        x, C = ctx.saved_tensors
        need_x, need_C = ctx.needs_input_grad[:2]
        dx, dC = F.kan_group_backward(x, C, dy.contiguous().float(), ctx.grid, need_dx=need_x,
                                      need_dC=need_C)
        if dx is not None and dx.dtype != x.dtype:
            dx = dx.to(x.dtype)
        if dC is not None and dC.dtype != C.dtype:
            dC = dC.to(C.dtype)
        return dx, dC, None, None, None


class KANGroupedActivation(torch.nn.Module):
    """Element-wise spline activation: channel ``i`` of ``[..., channels]``
    passes through cubic B-spline ``phi_{g(i)}``, shared by the consecutive
    channels of group ``g(i) = i * groups // channels``; ``groups ==
    channels`` gives one spline per channel.  Parameter ``coef [groups,
    grid_size + 3]``; output and gradients in float32."""

    def __init__(self, channels, groups=1, grid_size=8, grid_range=(-1.0, 1.0), dtype=torch.float32,
                 device=None, coef_std=0.1):
        super().__init__()
        if not 1 <= groups <= channels:
            raise ValueError("need 1 <= groups <= channels")
        self.channels = int(channels)
        self.groups = int(groups)
        self.grid_size = int(grid_size)
        self.grid_range = (float(grid_range[0]), float(grid_range[1]))
        self.coef = torch.nn.Parameter(torch.randn(groups, grid_size + 3, dtype=dtype, device=device) * coef_std)

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = _to_storage(x.reshape(-1, self.channels), self.coef.dtype).contiguous()
        y = GroupedFunction.apply(x2, self.coef, self.grid_range[0], self.grid_range[1], self.grid_size)
        return y.reshape(*lead, self.channels)

    def extra_repr(self):
        return "channels=%d, groups=%d, grid_size=%d, range=%s, dtype=%s" % (
            self.channels, self.groups, self.grid_size, self.grid_range, self.coef.dtype)


class SurfaceFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, C, lo, hi, G):
        ctx.grid = (lo, hi, G)
        ctx.save_for_backward(x, C)
        return F.kan_surface_forward(x, C, (lo, hi, G))

    @staticmethod
    def backward(ctx, dy):
        x, C = ctx.saved_tensors
        need_x, need_C = ctx.needs_input_grad[:2]
        dx, dC = F.kan_surface_backward(x, C, dy.contiguous().float(), ctx.grid, need_dx=need_x,
                                        need_dC=need_C)
        if dx is not None and dx.dtype != x.dtype:
            dx = dx.to(x.dtype)
        if dC is not None and dC.dtype != C.dtype:
            dC = dC.to(C.dtype)
        return dx, dC, None, None, None


class KANSurfaceLayer(torch.nn.Module):
    """2-D tensor-product spline layer: the inputs are taken in consecutive
    pairs ``(x[..., 2p], x[..., 2p+1])`` and output ``j`` sums a bicubic
    surface per pair, ``sum_{m,n} C[j, p, m, n] B_m(x1) B_n(x2)``.
    Parameter ``coef [out, in/2, grid_size + 3, grid_size + 3]``
    (``grid_size <= 13``); output and gradients in float32."""

    def __init__(self, in_features, out_features, grid_size=5, grid_range=(-1.0, 1.0), dtype=torch.float32,
                 device=None, coef_std=0.02):
        super().__init__()
        if in_features % 2:
            raise ValueError("the 2-D layer takes an even number of inputs")
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.grid_size = int(grid_size)
        self.grid_range = (float(grid_range[0]), float(grid_range[1]))
        K = grid_size + 3
        self.coef = torch.nn.Parameter(
            torch.randn(out_features, in_features // 2, K, K, dtype=dtype, device=device) * coef_std)

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = _to_storage(x.reshape(-1, self.in_features), self.coef.dtype).contiguous()
        y = SurfaceFunction.apply(x2, self.coef, self.grid_range[0], self.grid_range[1], self.grid_size)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return "in=%d (pairs=%d), out=%d, grid_size=%d, range=%s, dtype=%s" % (
            self.in_features, self.in_features // 2, self.out_features, self.grid_size, self.grid_range,
            self.coef.dtype)
