"""2-D tensor-product spline layer, float64, by the plain definition.

Test infrastructure (see ``oracle/__init__``).

The InKAN project page ("1D and 2D Splines") offers tensor-product B-spline
surfaces, beside the univariate spline layers, for approximating a function
of two inputs jointly.  The page gives no formula and no layout; this is the
reading the kernels follow.  The inputs of a row are taken in consecutive
pairs (x[b, 2p], x[b, 2p+1]), p = 0 .. P-1.  Every (output j, pair p) edge
carries one bicubic surface with coefficients C[j, p, m, n], m for the pair's
first input and n for its second, each over the layer's 1-D basis
(``bspline``; K = G + 3 functions), and output j sums its edges:

    y[b, j] = sum_p sum_{m,n} C[j, p, m, n] * B_m(x[b, 2p]) * B_n(x[b, 2p+1])

so each (row, pair) has at most 4 x 4 = 16 non-zero products.  Backward with
upstream ``dy [N, O]``:

    dx[b, 2p]     = sum_j dy[b, j] sum_{m,n} C[j, p, m, n] B'_m(x[b, 2p]) B_n(x[b, 2p+1])
    dx[b, 2p+1]   = sum_j dy[b, j] sum_{m,n} C[j, p, m, n] B_m(x[b, 2p]) B'_n(x[b, 2p+1])
    dC[j, p, m, n] = sum_b dy[b, j] B_m(x[b, 2p]) B_n(x[b, 2p+1])
"""

import numpy as np

from .bspline import basis, basis_derivative


def _pair_bases(x, lo, hi, G, d1=False, d2=False):
    x = np.asarray(x, dtype=np.float64)
    N, I = x.shape
    if I % 2:
        raise ValueError("the 2-D layer takes an even number of inputs")
    x1, x2 = x[:, 0::2], x[:, 1::2]
    B1 = (basis_derivative if d1 else basis)(x1, lo, hi, G)    # [N, P, K]
    B2 = (basis_derivative if d2 else basis)(x2, lo, hi, G)
    return B1, B2


def surface_forward(x, C, lo, hi, G):
    """``y [N, O]``; ``x [N, 2P]``, ``C [O, P, K, K]``."""
    C = np.asarray(C, dtype=np.float64)
    B1, B2 = _pair_bases(x, lo, hi, G)
    return np.einsum("npm,npq,jpmq->nj", B1, B2, C, optimize=True)


def surface_backward(x, C, dy, lo, hi, G):
    """``(dx [N, 2P], dC [O, P, K, K])``."""
    C = np.asarray(C, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    B1, B2 = _pair_bases(x, lo, hi, G)
    D1, D2 = _pair_bases(x, lo, hi, G, d1=True, d2=True)
    N, P, K = B1.shape
    dx = np.empty((N, 2 * P))
    dx[:, 0::2] = np.einsum("nj,npm,npq,jpmq->np", dy, D1, B2, C, optimize=True)
    dx[:, 1::2] = np.einsum("nj,npm,npq,jpmq->np", dy, B1, D2, C, optimize=True)
    dC = np.einsum("nj,npm,npq->jpmq", dy, B1, B2, optimize=True)
    return dx, dC


def surface_forward_rows(x, C, lo, hi, G, rows):
    """``y`` of the given rows only (rows depend only on their own inputs)."""
    return surface_forward(np.asarray(x)[rows], C, lo, hi, G)


def surface_coef_grad_pairs(x, dy, lo, hi, G, pairs):
    """``dC[j, p, :, :]`` for the given ``(j, p)`` pairs, each a sum over all
    rows: ``sum_b dy[b, j] * outer(B(x[b, 2p]), B(x[b, 2p+1]))``."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    out = []
    for j, p in pairs:
        B1 = basis(x[:, 2 * p], lo, hi, G)
        B2 = basis(x[:, 2 * p + 1], lo, hi, G)
        out.append(np.einsum("n,nm,nq->mq", dy[:, j], B1, B2))
    return np.stack(out)
