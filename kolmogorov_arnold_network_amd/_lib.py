"""ctypes view of the C ABI declared in ``include/kan.h``.

Argument marshalling only: structs, signatures and status codes.  Loading
fails loudly when the HIP library has not been built; there is no fallback.
"""

import ctypes
import os

from ._build import LIB_PATH

KAN_OK = 0
KAN_ERR_NULL = -1
KAN_ERR_SHAPE = -2
KAN_ERR_GRID = -3
KAN_ERR_DTYPE = -4
KAN_ERR_ALIGN = -5
KAN_ERR_WORKSPACE = -6
KAN_ERR_HIP = -7
KAN_ERR_UNSUPPORTED = -8
KAN_ERR_ALIAS = -9

KAN_F32 = 0
KAN_BF16 = 1

KAN_VARIANT_AUTO = 0
KAN_VARIANT_MFMA = 1
KAN_VARIANT_GATHER = 2

KAN_PASS_FORWARD = 0
KAN_PASS_BACKWARD = 1

KAN_FLAG_PREPARED = 1
KAN_FLAG_DENSE_FORWARD = 2
KAN_FLAG_TP_FORWARD = 4

KAN_STATIC_SCRATCH_BYTES = 32 << 20     # kan_forward_static's device array

ABI_VERSION = 1

# every symbol include/kan.h declares
EXPORTS = ("kan_abi_version", "kan_status_string", "kan_workspace_size", "kan_prepare",
           "kan_forward", "kan_forward_static", "kan_backward", "kan_basis_eval", "kan_basis_eval_tp", "kan_cast_f32_to_bf16",
           "kan_group_workspace_size", "kan_group_forward", "kan_group_backward",
           "kan_surface_workspace_size", "kan_surface_forward", "kan_surface_backward")


class kan_grid_t(ctypes.Structure):
    _fields_ = [("lo", ctypes.c_float), ("hi", ctypes.c_float),
                ("G", ctypes.c_int32), ("degree", ctypes.c_int32)]


class kan_desc_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("I", ctypes.c_int64), ("O", ctypes.c_int64),
                ("grid", kan_grid_t), ("dtype", ctypes.c_int32), ("has_base", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("flags", ctypes.c_int32)]


class kan_group_desc_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("I", ctypes.c_int64), ("groups", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("grid", kan_grid_t)]


class kan_surface_desc_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("P", ctypes.c_int64), ("O", ctypes.c_int64),
                ("grid", kan_grid_t), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class KanError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "HIP library %s is not built; run __graft_entry__.build() or "
            "python -m kolmogorov_arnold_network_amd._build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.kan_abi_version.restype = ctypes.c_int
    L.kan_abi_version.argtypes = []
    L.kan_status_string.restype = ctypes.c_char_p
    L.kan_status_string.argtypes = [ctypes.c_int]
    L.kan_workspace_size.restype = _sz
    L.kan_workspace_size.argtypes = [P(kan_desc_t), ctypes.c_int]
    L.kan_prepare.restype = ctypes.c_int
    L.kan_prepare.argtypes = [P(kan_desc_t), ctypes.c_int, _vp, _vp, _vp, _vp, _sz, _vp]
    L.kan_forward.restype = ctypes.c_int
    L.kan_forward.argtypes = [P(kan_desc_t), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.kan_forward_static.restype = ctypes.c_int
    L.kan_forward_static.argtypes = [P(kan_desc_t), _vp, _vp, _vp, _vp, _vp]
    L.kan_backward.restype = ctypes.c_int
    L.kan_backward.argtypes = [P(kan_desc_t), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    for f in (L.kan_basis_eval, L.kan_basis_eval_tp):
        f.restype = ctypes.c_int
        f.argtypes = [P(kan_grid_t), _i64, ctypes.c_int, _vp, _vp, _vp, _vp]
    L.kan_group_workspace_size.restype = _sz
    L.kan_group_workspace_size.argtypes = [P(kan_group_desc_t)]
    L.kan_group_forward.restype = ctypes.c_int
    L.kan_group_forward.argtypes = [P(kan_group_desc_t), _vp, _vp, _vp, _vp]
    L.kan_group_backward.restype = ctypes.c_int
    L.kan_group_backward.argtypes = [P(kan_group_desc_t), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.kan_surface_workspace_size.restype = _sz
    L.kan_surface_workspace_size.argtypes = [P(kan_surface_desc_t), ctypes.c_int]
    L.kan_surface_forward.restype = ctypes.c_int
    L.kan_surface_forward.argtypes = [P(kan_surface_desc_t), _vp, _vp, _vp, _vp, _sz, _vp]
    L.kan_surface_backward.restype = ctypes.c_int
    L.kan_surface_backward.argtypes = [P(kan_surface_desc_t), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.kan_cast_f32_to_bf16.restype = ctypes.c_int
    L.kan_cast_f32_to_bf16.argtypes = [_vp, _vp, _i64, _vp]
    if L.kan_abi_version() != ABI_VERSION:
        raise RuntimeError("libkan ABI version %d, binding expects %d"
                           % (L.kan_abi_version(), ABI_VERSION))
    _lib = L
    return L


def status_string(status):
    return lib().kan_status_string(int(status)).decode()


def check(status, what):
    if status != KAN_OK:
        raise KanError(status, what)
    return status


def make_desc(N, I, O, lo, hi, G, dtype, has_base, variant=KAN_VARIANT_AUTO, flags=0, degree=3):
    d = kan_desc_t()
    d.N, d.I, d.O = int(N), int(I), int(O)
    d.grid.lo, d.grid.hi, d.grid.G, d.grid.degree = float(lo), float(hi), int(G), int(degree)
    d.dtype, d.has_base, d.variant, d.flags = int(dtype), int(has_base), int(variant), int(flags)
    return d


def make_group_desc(N, I, groups, lo, hi, G, dtype, degree=3):
    d = kan_group_desc_t()
    d.N, d.I, d.groups, d.dtype = int(N), int(I), int(groups), int(dtype)
    d.grid.lo, d.grid.hi, d.grid.G, d.grid.degree = float(lo), float(hi), int(G), int(degree)
    return d


def make_surface_desc(N, P, O, lo, hi, G, dtype, degree=3, flags=0):
    d = kan_surface_desc_t()
    d.N, d.P, d.O, d.dtype, d.flags = int(N), int(P), int(O), int(dtype), int(flags)
    return _fill_grid(d, lo, hi, G, degree)


def _fill_grid(d, lo, hi, G, degree):
    d.grid.lo, d.grid.hi, d.grid.G, d.grid.degree = float(lo), float(hi), int(G), int(degree)
    return d
