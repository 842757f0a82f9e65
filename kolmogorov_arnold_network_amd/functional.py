"""Torch-facing wrappers of the C entry points, under the same names.

Each wrapper checks dtype / device / contiguity, allocates the outputs and the
workspace with torch (device memory only), and passes raw pointers plus the
current HIP stream to the library.  No arithmetic of the layer happens here.
"""

import ctypes

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.KAN_F32, torch.bfloat16: L.KAN_BF16}
_VARIANTS = {"auto": L.KAN_VARIANT_AUTO, "mfma": L.KAN_VARIANT_MFMA, "gather": L.KAN_VARIANT_GATHER}


def _variant(v):
    return _VARIANTS[v] if isinstance(v, str) else int(v)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_tensor(t, name, dtypes, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _check_out(t, name, shape, device):
    """A caller's output tensor: float32, contiguous, on ``device``, of ``shape``."""
    _check_tensor(t, name, (torch.float32,), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_ws(ws, device):
    """A caller's ``(buffer, bytes)`` workspace: the buffer must hold the bytes
    it declares (the library trusts the declared size)."""
    buf, n = ws
    n = int(n)
    if n < 0:
        raise ValueError("workspace size must be >= 0")
    if n > 0:
        if buf is None or not buf.is_cuda or buf.device != device or not buf.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor on %s" % device)
        if buf.numel() * buf.element_size() < n:
            raise ValueError("workspace holds %d bytes, %d declared"
                             % (buf.numel() * buf.element_size(), n))
    return buf, n


def layer_desc(x, C, W, grid, variant="auto", flags=0):
    """``kan_desc_t`` for ``x [N, I]``, ``C [O, I, G+D]``, ``W [O, I]`` or None;
    the spline degree D (1 .. 5, 3 for the pages' cubic layer) is read off C."""
    lo, hi, G = grid
    N, I = x.shape
    O, I2, K = C.shape
    if I2 != I or not 1 <= K - G <= 5:
        raise ValueError("C must be [O, I, G+D] = [%d, %d, %d+D], D in 1..5, got %s"
                         % (O, I, G, tuple(C.shape)))
    if W is not None and tuple(W.shape) != (O, I):
        raise ValueError("W_base must be [O, I]")
    if x.dtype != C.dtype or (W is not None and W.dtype != C.dtype):
        raise ValueError("x, C and W_base must share one dtype")
    return L.make_desc(N, I, O, lo, hi, G, _DTYPES[x.dtype], W is not None, _variant(variant), flags,
                       degree=K - G)


def kan_workspace_size(desc, pass_):
    n = L.lib().kan_workspace_size(ctypes.byref(desc), int(pass_))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid layer description")
    return int(n)


def workspace(desc, pass_, device):
    """A fresh device workspace for one pass (torch allocator; 512-byte aligned)."""
    n = kan_workspace_size(desc, pass_)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def _fwd_flags(dense_forward, tp_forward):
    return (L.KAN_FLAG_DENSE_FORWARD if dense_forward else 0) | (L.KAN_FLAG_TP_FORWARD if tp_forward else 0)


def kan_prepare(x, C, W, grid, pass_, dy=None, variant="auto", ws=None, dense_forward=False, tp_forward=False):
    """Packs the pass's operands into a workspace; returns ``(ws, ws_bytes)``."""
    _check_tensor(C, "C", _DTYPES)
    _check_tensor(W, "W_base", _DTYPES, C.device)
    _check_tensor(dy, "dy", (torch.float32,), C.device)
    desc = layer_desc(x, C, W, grid, variant, _fwd_flags(dense_forward, tp_forward))
    if dy is not None and tuple(dy.shape) != (x.shape[0], C.shape[0]):
        raise ValueError("dy must be [N, O]")
    if ws is None:
        ws = workspace(desc, pass_, C.device)
    buf, n = _check_ws(ws, C.device)
    L.check(L.lib().kan_prepare(ctypes.byref(desc), int(pass_), _ptr(C), _ptr(W), _ptr(dy),
                                _ptr(buf), n, _stream(C)), "kan_prepare")
    return ws


def kan_forward(x, C, W, grid, variant="auto", ws=None, prepared=False, out=None,
                dense_forward=False, tp_forward=False):
    """``y [N, O]`` float32 of one KAN layer.  ``dense_forward`` turns off the
    structured-sparse forward of bf16 layers (``KAN_FLAG_DENSE_FORWARD``);
    ``tp_forward`` generates the dense bf16 basis tile by the truncated-power
    form (``KAN_FLAG_TP_FORWARD``)."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    _check_tensor(W, "W_base", _DTYPES, x.device)
    flags = (L.KAN_FLAG_PREPARED if prepared else 0) | _fwd_flags(dense_forward, tp_forward)
    desc = layer_desc(x, C, W, grid, variant, flags)
    if ws is None:
        ws = workspace(desc, L.KAN_PASS_FORWARD, x.device)
    buf, n = _check_ws(ws, x.device)
    y = out if out is not None else torch.empty((x.shape[0], C.shape[0]), dtype=torch.float32,
                                                device=x.device)
    _check_out(y, "y", (x.shape[0], C.shape[0]), x.device)
    L.check(L.lib().kan_forward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(W), _ptr(y), _ptr(buf),
                                n, _stream(x)), "kan_forward")
    return y


def kan_forward_static(x, C, W, grid, variant="auto", out=None, dense_forward=False):
    """``y [N, O]`` float32 of one KAN layer with the library's own static
    device workspace (no workspace argument, nothing allocated but ``y``
    when ``out`` is not given)."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    _check_tensor(W, "W_base", _DTYPES, x.device)
    desc = layer_desc(x, C, W, grid, variant, L.KAN_FLAG_DENSE_FORWARD if dense_forward else 0)
    y = out if out is not None else torch.empty((x.shape[0], C.shape[0]), dtype=torch.float32,
                                                device=x.device)
    _check_out(y, "y", (x.shape[0], C.shape[0]), x.device)
    L.check(L.lib().kan_forward_static(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(W), _ptr(y), _stream(x)),
            "kan_forward_static")
    return y


def kan_backward(x, C, W, dy, grid, need_dx=True, need_dC=True, need_dW=True, variant="auto",
                 ws=None, prepared=False):
    """``(dx [N, I], dC [O, I, G+3], dW_base [O, I])`` float32; unrequested ones are None."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    _check_tensor(W, "W_base", _DTYPES, x.device)
    _check_tensor(dy, "dy", (torch.float32,), x.device)
    desc = layer_desc(x, C, W, grid, variant, L.KAN_FLAG_PREPARED if prepared else 0)
    if tuple(dy.shape) != (x.shape[0], C.shape[0]):
        raise ValueError("dy must be [N, O]")
    if ws is None:
        ws = workspace(desc, L.KAN_PASS_BACKWARD, x.device)
    buf, n = _check_ws(ws, x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty(x.shape, **f32) if need_dx else None
    dC = torch.empty(C.shape, **f32) if need_dC else None
    dW = torch.empty(W.shape, **f32) if (need_dW and W is not None) else None
    L.check(L.lib().kan_backward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(W), _ptr(dy), _ptr(dx),
                                 _ptr(dC), _ptr(dW), _ptr(buf), n, _stream(x)), "kan_backward")
    return dx, dC, dW


def _basis(fn, name, x, grid, need_B, need_dB, degree):
    _check_tensor(x, "x", _DTYPES)
    lo, hi, G = grid
    g = L.kan_grid_t(float(lo), float(hi), int(G), int(degree))
    n = x.numel()
    B = torch.empty((n, G + degree), dtype=torch.float32, device=x.device) if need_B else None
    dB = torch.empty((n, G + degree), dtype=torch.float32, device=x.device) if need_dB else None
    L.check(fn(ctypes.byref(g), n, _DTYPES[x.dtype], _ptr(x), _ptr(B), _ptr(dB), _stream(x)), name)
    return B, dB


def kan_basis_eval(x, grid, need_B=True, need_dB=True, degree=3):
    """Dense ``B [n, G+degree]`` and ``dB`` of a 1-D tensor of inputs (local span form)."""
    return _basis(L.lib().kan_basis_eval, "kan_basis_eval", x, grid, need_B, need_dB, degree)


def kan_basis_eval_tp(x, grid, need_B=True, need_dB=True, degree=3):
    """The same, from the truncated-power form (every basis function on its own)."""
    return _basis(L.lib().kan_basis_eval_tp, "kan_basis_eval_tp", x, grid, need_B, need_dB, degree)


def group_desc(x, C, grid):
    """``kan_group_desc_t`` for ``x [N, I]`` and ``C [groups, G+3]``."""
    lo, hi, G = grid
    if x.dim() != 2 or C.dim() != 2 or C.shape[1] != G + 3:
        raise ValueError("x must be [N, I] and C [groups, G+3]")
    if x.dtype != C.dtype:
        raise ValueError("x and C must share one dtype")
    return L.make_group_desc(x.shape[0], x.shape[1], C.shape[0], lo, hi, G, _DTYPES[x.dtype])


def kan_group_workspace_size(desc):
    n = L.lib().kan_group_workspace_size(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid grouped activation description")
    return int(n)


def kan_group_forward(x, C, grid, out=None):
    """``y [N, I]`` float32 of the grouped spline activation
    ``y[b, i] = sum_m C[g(i), m] B_m(x[b, i])``, ``g(i) = i * groups // I``."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    desc = group_desc(x, C, grid)
    y = out if out is not None else torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _check_out(y, "y", x.shape, x.device)
    L.check(L.lib().kan_group_forward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(y), _stream(x)),
            "kan_group_forward")
    return y


def kan_group_backward(x, C, dy, grid, need_dx=True, need_dC=True, ws=None):
    """``(dx [N, I], dC [groups, G+3])`` float32; unrequested ones are None."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    _check_tensor(dy, "dy", (torch.float32,), x.device)
    desc = group_desc(x, C, grid)
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must be [N, I]")
    if ws is None:
        n = kan_group_workspace_size(desc) if need_dC else 0
        ws = (torch.empty(max(n, 1), dtype=torch.uint8, device=x.device), n)
    buf, n = _check_ws(ws, x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty(x.shape, **f32) if need_dx else None
    dC = torch.empty(C.shape, **f32) if need_dC else None
    L.check(L.lib().kan_group_backward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(dy), _ptr(dx),
                                       _ptr(dC), _ptr(buf), n, _stream(x)), "kan_group_backward")
    return dx, dC


def surface_desc(x, C, grid):
    """``kan_surface_desc_t`` for ``x [N, 2P]`` and ``C [O, P, G+3, G+3]``."""
    lo, hi, G = grid
    if x.dim() != 2 or x.shape[1] % 2 or C.dim() != 4:
        raise ValueError("x must be [N, 2P] and C [O, P, G+3, G+3]")
    O, P, K1, K2 = C.shape
    if 2 * P != x.shape[1] or K1 != G + 3 or K2 != G + 3:
        raise ValueError("C must be [O, %d, %d, %d], got %s" % (x.shape[1] // 2, G + 3, G + 3, tuple(C.shape)))
    if x.dtype != C.dtype:
        raise ValueError("x and C must share one dtype")
    return L.make_surface_desc(x.shape[0], P, O, lo, hi, G, _DTYPES[x.dtype])


def kan_surface_workspace_size(desc, pass_):
    n = L.lib().kan_surface_workspace_size(ctypes.byref(desc), int(pass_))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid 2-D layer description")
    return int(n)


def _surface_ws(desc, pass_, device):
    n = kan_surface_workspace_size(desc, pass_)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def kan_surface_forward(x, C, grid, ws=None, out=None, dense_forward=False):
    """``y [N, O]`` float32 of the 2-D tensor-product layer
    ``y[b, j] = sum_p sum_{m,n} C[j, p, m, n] B_m(x[b, 2p]) B_n(x[b, 2p+1])``;
    ``dense_forward`` turns off the structured-sparse forward (bf16, G = 5)."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    desc = surface_desc(x, C, grid)
    if dense_forward:
        desc.flags = L.KAN_FLAG_DENSE_FORWARD
    buf, n = _check_ws(ws if ws is not None else _surface_ws(desc, L.KAN_PASS_FORWARD, x.device), x.device)
    y = out if out is not None else torch.empty((x.shape[0], C.shape[0]), dtype=torch.float32,
                                                device=x.device)
    _check_out(y, "y", (x.shape[0], C.shape[0]), x.device)
    L.check(L.lib().kan_surface_forward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(y), _ptr(buf), n,
                                        _stream(x)), "kan_surface_forward")
    return y


def kan_surface_backward(x, C, dy, grid, need_dx=True, need_dC=True, ws=None):
    """``(dx [N, 2P], dC [O, P, G+3, G+3])`` float32; unrequested ones are None."""
    _check_tensor(x, "x", _DTYPES)
    _check_tensor(C, "C", _DTYPES, x.device)
    _check_tensor(dy, "dy", (torch.float32,), x.device)
    desc = surface_desc(x, C, grid)
    if tuple(dy.shape) != (x.shape[0], C.shape[0]):
        raise ValueError("dy must be [N, O]")
    buf, n = _check_ws(ws if ws is not None else _surface_ws(desc, L.KAN_PASS_BACKWARD, x.device), x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty(x.shape, **f32) if need_dx else None
    dC = torch.empty(C.shape, **f32) if need_dC else None
    L.check(L.lib().kan_surface_backward(ctypes.byref(desc), _ptr(x), _ptr(C), _ptr(dy), _ptr(dx), _ptr(dC),
                                         _ptr(buf), n, _stream(x)), "kan_surface_backward")
    return dx, dC


def kan_cast_f32_to_bf16(t, out=None):
    """Round-to-nearest-even float32 -> bfloat16 on the device."""
    _check_tensor(t, "input", (torch.float32,))
    o = out if out is not None else torch.empty(t.shape, dtype=torch.bfloat16, device=t.device)
    L.check(L.lib().kan_cast_f32_to_bf16(_ptr(t), _ptr(o), t.numel(), _stream(t)),
            "kan_cast_f32_to_bf16")
    return o
