"""Plain float64 CPU oracle for the B-spline Kolmogorov-Arnold Network layer.

TEST INFRASTRUCTURE ONLY.  This package states, as directly as NumPy allows,
what the KAN layer computes, so that the HIP path can be checked against it.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product package never imports it, and it
imports nothing from the product package: the two share no code.

Contents
--------
``bspline``  knot vector, Cox-de Boor recursion, basis derivatives.
``layer``    single KAN layer forward / backward, two-layer networks,
             sampled gradients for large shapes.
``bf16``     round-to-nearest-even cast of float32 to bfloat16.
``grouped``  per-channel (grouped) spline activation forward / backward.
``surface``  2-D tensor-product spline layer (pairs of inputs) forward /
             backward, and sampled helpers for large shapes.

Every function cites the passage of the pages it follows.  Pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle.py``, ``test_oracle_grouped.py``
and ``test_oracle_surface.py``; there is no function here whose parity is
unpinned.
"""

from .bspline import knots, cox_de_boor, basis, basis_derivative, n_basis
from .layer import (silu, silu_prime, layer_forward, layer_backward,
                    layer_forward_rows, layer_backward_rows,
                    coef_grad_pairs, network_forward, network_backward)
from .bf16 import round_bf16
from .grouped import group_of, grouped_forward, grouped_backward
from .surface import (surface_forward, surface_backward, surface_forward_rows,
                      surface_coef_grad_pairs)

__all__ = [
    "knots", "cox_de_boor", "basis", "basis_derivative", "n_basis",
    "silu", "silu_prime", "layer_forward", "layer_backward",
    "layer_forward_rows", "layer_backward_rows", "coef_grad_pairs",
    "network_forward", "network_backward", "round_bf16",
    "group_of", "grouped_forward", "grouped_backward",
    "surface_forward", "surface_backward", "surface_forward_rows", "surface_coef_grad_pairs",
]
