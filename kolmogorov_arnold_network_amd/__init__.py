"""MI355X (gfx950) B-spline Kolmogorov-Arnold Network layer.

The layer computes ``y[b, j] = sum_i sum_m C[j, i, m] B_m(x[b, i])`` (plus an
optional ``W_base silu(x)`` branch) with uniform cubic B-splines on an
extended knot grid, and its training backward (dx, dC, dW_base).  All of it
runs in hand-written HIP kernels behind the C ABI of ``include/kan.h``; so
does the grouped (per-channel) spline activation ``y[b, i] = phi_{g(i)}(x[b, i])``
and its backward, and the 2-D tensor-product spline layer over pairs of
inputs.  This
package binds that ABI (``functional``) and wraps it as torch modules
(``modules``).
"""

from . import _lib
from .functional import (kan_forward, kan_forward_static, kan_backward, kan_prepare, kan_basis_eval, kan_basis_eval_tp,
                         kan_cast_f32_to_bf16, kan_workspace_size, layer_desc, workspace,
                         kan_group_forward, kan_group_backward, kan_group_workspace_size, group_desc,
                         kan_surface_forward, kan_surface_backward, kan_surface_workspace_size,
                         surface_desc)
from .modules import (KANLayer, KANNetwork, KANFunction, KANGroupedActivation, KANSurfaceLayer,
                      GroupedFunction, SurfaceFunction)

__all__ = ["kan_forward", "kan_forward_static", "kan_backward", "kan_prepare", "kan_basis_eval", "kan_basis_eval_tp",
           "kan_cast_f32_to_bf16",
           "kan_workspace_size", "layer_desc", "workspace", "KANLayer", "KANNetwork", "KANFunction",
           "kan_group_forward", "kan_group_backward", "kan_group_workspace_size", "group_desc",
           "kan_surface_forward", "kan_surface_backward", "kan_surface_workspace_size", "surface_desc",
           "KANGroupedActivation", "KANSurfaceLayer", "GroupedFunction", "SurfaceFunction"]
