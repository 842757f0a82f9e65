"""KAN layer forward and training backward, float64, by the plain definition.

Test infrastructure (see ``oracle/__init__``).

Layer definition (InKAN project page, "What is a KAN?"): output ``j`` is a sum
over inputs ``i`` of one learned univariate function per edge,
``y_j = sum_i phi_ji(x_i)``, and each ``phi_ji`` is a cubic B-spline, so

    y[b, j] = sum_i sum_m C[j, i, m] * B_m(x[b, i])
              (+ sum_i W_base[j, i] * silu(x[b, i])   if the base branch is on)

There is no bias term (the KAN formula on that page has none).  The optional
residual ``W_base * silu(x)`` branch is not on the pages; this library offers
it as an option and the oracle states it here the same way.

Shapes: ``x [N, I]``, ``C [O, I, K]`` with ``K = G + 3`` and ``m`` fastest,
``W_base [O, I]`` (or ``None``), ``y``/``dy [N, O]``.  The layer functions
also take a spline degree ``k`` (default 3, the pages' cubic layer); for the
degree-``k`` form the FlashKAN page states for its basis, ``K = G + k`` on a
grid extended by ``k`` knots per side (``bspline``).

Training backward ("same optimizer, same training loop", InKAN page, "Why
InKAN?" and "Quick Start"): with upstream gradient ``dy``,

    dx[b, i]      = sum_j dy[b, j] * ( sum_m C[j, i, m] * B'_m(x[b, i])
                                       + W_base[j, i] * silu'(x[b, i]) )
    dC[j, i, m]   = sum_b dy[b, j] * B_m(x[b, i])
    dW_base[j, i] = sum_b dy[b, j] * silu(x[b, i])

Inputs outside the extended knot grid get ``B_m = 0`` for every ``m`` (the
exact B-splines of the knot vector are used everywhere); no clamp of ``x``
happens inside the layer.
"""

import numpy as np

from .bspline import basis, basis_derivative
from .bf16 import round_bf16


def silu(x):
    """``silu(x) = x * sigmoid(x) = x / (1 + exp(-x))``."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def silu_prime(x):
    """``d silu / dx = s (1 + x (1 - s))`` with ``s = sigmoid(x)``."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def layer_forward(x, C, W, lo, hi, G, k=3):
    """``y [N, O]`` of one KAN layer (``W`` may be ``None``: no base branch)."""
    x, C, W = _f64(x), _f64(C), _f64(W)
    N, I = x.shape
    O, I2, K = C.shape
    assert I2 == I and K == G + k
    B = basis(x, lo, hi, G, k)                   # [N, I, K]
    # sum over the pair (i, m), written as one product over the flattened index
    y = B.reshape(N, I * K) @ C.reshape(O, I * K).T
    if W is not None:
        y = y + silu(x) @ W.T
    return y


def layer_backward(x, C, W, dy, lo, hi, G, need=("dx", "dC", "dW"), k=3):
    """``(dx, dC, dW)`` of one KAN layer; entries not in ``need`` are ``None``.

    ``dW`` is ``None`` as well when ``W`` is ``None``.
    """
    x, C, W, dy = _f64(x), _f64(C), _f64(W), _f64(dy)
    N, I = x.shape
    O, _, K = C.shape
    dx = dC = dW = None
    if "dx" in need:
        dB = basis_derivative(x, lo, hi, G, k)   # [N, I, K]
        # P[b, i, m] = sum_j dy[b, j] C[j, i, m]
        P = (dy @ C.reshape(O, I * K)).reshape(N, I, K)
        dx = np.sum(P * dB, axis=2)
        if W is not None:
            dx = dx + (dy @ W) * silu_prime(x)
    if "dC" in need:
        B = basis(x, lo, hi, G, k)
        dC = (dy.T @ B.reshape(N, I * K)).reshape(O, I, K)
    if "dW" in need and W is not None:
        dW = dy.T @ silu(x)
    return dx, dC, dW


def layer_forward_rows(x, C, W, lo, hi, G, rows):
    """``y`` on a subset of rows: rows of ``y`` depend only on the same rows of ``x``."""
    return layer_forward(np.asarray(x)[rows], C, W, lo, hi, G)


def layer_backward_rows(x, C, W, dy, lo, hi, G, rows):
    """``dx`` on a subset of rows (a row of ``dx`` needs only that row of ``x`` and ``dy``)."""
    dx, _, _ = layer_backward(np.asarray(x)[rows], C, W, np.asarray(dy)[rows],
                              lo, hi, G, need=("dx",))
    return dx


def coef_grad_pairs(x, dy, pairs, lo, hi, G, with_base):
    """``dC[j, i, :]`` and ``dW_base[j, i]`` for the listed ``(j, i)`` pairs.

    Each is its own sum over every row ``b``, so a pair needs only column
    ``i`` of ``x`` and column ``j`` of ``dy``.  Returns ``(dC_pairs [P, K],
    dW_pairs [P] or None)``.
    """
    x = np.asarray(x)
    dy = np.asarray(dy)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    K = G + 3
    dCp = np.zeros((len(pairs), K))
    dWp = np.zeros(len(pairs)) if with_base else None
    cache = {}
    for p, (j, i) in enumerate(pairs):
        if i not in cache:
            xi = x[:, i].astype(np.float64)
            cache[i] = (basis(xi, lo, hi, G), silu(xi))
        Bi, si = cache[i]
        dyj = dy[:, j].astype(np.float64)
        dCp[p] = dyj @ Bi
        if with_base:
            dWp[p] = dyj @ si
    return dCp, dWp


def network_forward(x, layers, lo, hi, G, bf16_between=False, k=3):
    """Activations of a chain of KAN layers.

    ``layers`` is a list of ``(C, W_base)``.  Layers compose with nothing in
    between (the InKAN "Quick Start" network is a plain chain of layers).
    With ``bf16_between`` the float output of each hidden layer is rounded to
    bfloat16 before the next layer reads it, as the bf16 network does.
    Returns ``[x0, x1, ..., y]`` where ``x_{l+1}`` is the input of layer ``l+1``.
    """
    acts = [np.asarray(x, dtype=np.float64)]
    for li, (C, W) in enumerate(layers):
        y = layer_forward(acts[-1], C, W, lo, hi, G, k=k)
        if bf16_between and li + 1 < len(layers):
            y = round_bf16(y)
        acts.append(y)
    return acts


def network_backward(acts, layers, dy, lo, hi, G, k=3):
    """Gradients of a chain of KAN layers by the chain rule.

    ``acts`` is the output of ``network_forward``.  A rounding cast between
    layers passes the gradient through unchanged.  Returns ``(dx0, grads)``
    with ``grads[l] = (dC_l, dW_l)``.
    """
    grads = [None] * len(layers)
    g = np.asarray(dy, dtype=np.float64)
    for li in range(len(layers) - 1, -1, -1):
        C, W = layers[li]
        dx, dC, dW = layer_backward(acts[li], C, W, g, lo, hi, G, k=k)
        grads[li] = (dC, dW)
        g = dx
    return g, grads
