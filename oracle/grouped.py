"""Per-channel (grouped) spline activation, float64, by the plain definition.

Test infrastructure (see ``oracle/__init__``).

The element-wise form of the KAN edge function: channel ``i`` of a row passes
through one learned cubic B-spline, shared by the channels of its group,

    y[b, i] = sum_m C[g(i), m] * B_m(x[b, i]),     g(i) = i * groups // I,

so the ``I`` channels form ``groups`` blocks of consecutive channels (``groups
= I``: one spline per channel, "per-coordinate spline curves" on the InKAN
project page; fewer groups: the grouped activations of KAT, whose training
slowdown the FlashKAT abstract traces to the accumulation of the coefficient
gradient).  ``C [groups, K]``, ``K = G + 3``; the basis is that of the layer
(``bspline``).  Backward with upstream ``dy [N, I]``:

    dx[b, i]  = dy[b, i] * sum_m C[g(i), m] * B'_m(x[b, i])
    dC[g, m]  = sum_b sum_{i in g} dy[b, i] * B_m(x[b, i])
"""

import numpy as np

from .bspline import basis, basis_derivative


def group_of(I, groups):
    """``g(i)`` for every channel: blocks of consecutive channels."""
    return (np.arange(I) * groups) // I


def grouped_forward(x, C, lo, hi, G):
    """``y [N, I]``; ``C [groups, K]``."""
    x = np.asarray(x, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N, I = x.shape
    g = group_of(I, C.shape[0])
    B = basis(x, lo, hi, G)                          # [N, I, K]
    return np.einsum("nik,ik->ni", B, C[g])


def grouped_backward(x, C, dy, lo, hi, G):
    """``(dx [N, I], dC [groups, K])``."""
    x = np.asarray(x, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    N, I = x.shape
    groups, K = C.shape
    g = group_of(I, groups)
    dB = basis_derivative(x, lo, hi, G)
    dx = dy * np.einsum("nik,ik->ni", dB, C[g])
    B = basis(x, lo, hi, G)
    per_channel = np.einsum("ni,nik->ik", dy, B)     # [I, K]
    dC = np.zeros((groups, K))
    np.add.at(dC, g, per_channel)
    return dx, dC
