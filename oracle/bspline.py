"""B-spline basis on an extended uniform knot grid, by the Cox-de Boor recursion.

Test infrastructure (see ``oracle/__init__``).  float64, NumPy only.

Sources on the pages:
* InKAN project page, "What is a KAN?": each edge function is a learned
  cubic B-spline with local support (one coefficient moves the curve over
  about 4 knot intervals).
* mlsift "GPU kernel" listing, FlashKAN entry: the standard evaluation is the
  Cox-de Boor recursion, k sequential passes for degree k; it is the slow
  baseline that faster forms are compared against.
* InKAN project page, "Performance" table: "Cox-de Boor (recursive)" is the
  1.0x reference and grid sizes are 8, 20, 50.

Reading taken where the pages are silent: the grid has ``G`` equal intervals
on ``[lo, hi]`` and is extended by ``k`` knots on each side, so a degree-``k``
spline has ``G + k`` basis functions; degree-0 pieces use half-open intervals
``[t_r, t_{r+1})``.  With ``k = 3`` this gives ``G + 7`` knots and ``G + 3``
cubic basis functions (11 at ``G = 8``).
"""

import numpy as np


def knots(lo, hi, G, k=3):
    """Extended uniform knot vector ``t_r = lo + (r - k) h``, ``r = 0 .. G + 2k``.

    ``h = (hi - lo) / G``.  The interior knots ``t_k .. t_{G+k}`` split
    ``[lo, hi]`` into ``G`` intervals; ``k`` more knots continue the grid on
    each side so that every point of ``[lo, hi]`` is covered by ``k + 1``
    basis functions.
    """
    if not (G >= 1 and k >= 0 and hi > lo):
        raise ValueError("need G >= 1, k >= 0, hi > lo")
    h = (float(hi) - float(lo)) / G
    r = np.arange(G + 2 * k + 1, dtype=np.float64)
    return float(lo) + (r - k) * h


def n_basis(G, k=3):
    """Number of degree-k basis functions on the extended grid: ``G + k``."""
    return G + k


def cox_de_boor(x, t, p):
    """All degree-``p`` B-splines ``B_{r,p}(x)`` on knot vector ``t``.

    The textbook recursion, one pass per degree (the "k sequential passes" of
    the FlashKAN entry):

        B_{r,0}(x) = 1 if t_r <= x < t_{r+1} else 0
        B_{r,q}(x) = (x - t_r) / (t_{r+q} - t_r) * B_{r,q-1}(x)
                   + (t_{r+q+1} - x) / (t_{r+q+1} - t_{r+1}) * B_{r+1,q-1}(x)

    with a term dropped when its denominator is zero.  Returns an array of
    shape ``x.shape + (len(t) - p - 1,)``.
    """
    x = np.asarray(x, dtype=np.float64)[..., None]
    t = np.asarray(t, dtype=np.float64)
    # degree 0: indicator of the half-open knot interval
    B = ((t[:-1] <= x) & (x < t[1:])).astype(np.float64)
    for q in range(1, p + 1):
        n = len(t) - q - 1                     # number of degree-q functions
        den_l = t[q:q + n] - t[:n]             # t_{r+q} - t_r
        den_r = t[q + 1:q + 1 + n] - t[1:1 + n]  # t_{r+q+1} - t_{r+1}
        wl = np.where(den_l > 0, (x - t[:n]) / np.where(den_l > 0, den_l, 1.0), 0.0)
        wr = np.where(den_r > 0, (t[q + 1:q + 1 + n] - x) / np.where(den_r > 0, den_r, 1.0), 0.0)
        B = wl * B[..., :n] + wr * B[..., 1:n + 1]
    return B


def basis(x, lo, hi, G, k=3):
    """``B_m(x)``, ``m = 0 .. G + k - 1``, degree ``k`` on the extended grid."""
    return cox_de_boor(x, knots(lo, hi, G, k), k)


def basis_derivative(x, lo, hi, G, k=3):
    """``d B_m / dx``, ``m = 0 .. G + k - 1``.

    The textbook derivative of a B-spline in terms of one degree lower,

        B'_{m,k}(x) = k / (t_{m+k} - t_m) * B_{m,k-1}(x)
                    - k / (t_{m+k+1} - t_{m+1}) * B_{m+1,k-1}(x),

    with the degree ``k - 1`` functions taken from the same recursion stopped
    one pass early.  All ``G + k + 1`` of them are used: the last one is
    supported on ``[hi, hi + k h)`` and matters for inputs past ``hi``.
    """
    t = knots(lo, hi, G, k)
    if k == 0:
        return np.zeros(np.shape(x) + (G,))
    Bl = cox_de_boor(x, t, k - 1)              # G + k + 1 functions
    n = G + k
    den_l = t[k:k + n] - t[:n]
    den_r = t[k + 1:k + 1 + n] - t[1:1 + n]
    return k / den_l * Bl[..., :n] - k / den_r * Bl[..., 1:n + 1]
