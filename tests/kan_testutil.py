"""Helpers shared by the tests: error metrics, loading the library, device copies."""

import os

import numpy as np

TOL_F32 = 1e-5      # normwise max relative error, float32 path
TOL_BF16 = 1e-2     # relative Frobenius error, bf16-input / float32-accumulate path


def rel_inf(a, r):
    """max |a - r| / max |r| (absolute when r is all zero)."""
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if a.size == 0:
        return 0.0
    d = float(np.max(np.abs(a - r)))
    m = float(np.max(np.abs(r)))
    return d / m if m > 0 else d


def rel_fro(a, r):
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n = float(np.linalg.norm(r))
    return float(np.linalg.norm(a - r)) / n if n > 0 else float(np.linalg.norm(a))


def metric(dtype):
    return (rel_inf, TOL_F32) if dtype == "f32" else (rel_fro, TOL_BF16)


def ensure_built():
    """Load the library, compiling it first only if nothing is built yet."""
    from kolmogorov_arnold_network_amd import _build, _lib
    if not os.path.exists(_build.LIB_PATH):
        _build.build_library()
    return _lib.lib()


def to_dev(a, dtype_name, device="cuda:0"):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype_name == "bf16" else t
