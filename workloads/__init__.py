"""Seeded synthetic inputs for the KAN layer workloads.

This module only draws random numbers and casts them to the storage dtype; it
holds none of the layer's arithmetic.  It is the one module that both the HIP
path's tests/benchmark and the CPU oracle read, so that both see the same
bits.  Nothing here imports the oracle or the product package.

Workloads (shapes follow the pages' own examples):

* ``c1``  one layer 8 -> 4, batch 32, float32, G = 8 on [-1, 1], no base
  branch (the InKAN "Quick Start" single layer); x ~ U(-1, 1) clamped to
  [-1, 1]; C ~ N(0, 0.1); dy ~ N(0, 1).
* ``c2``  two layers 784 -> 64 -> 10, batch 1024, float32, G = 8, base branch
  (the InKAN "Quick Start" network); x ~ N(0, 0.5) clamped to [-1, 1];
  C ~ N(0, 0.1); W_base ~ N(0, 1/sqrt(in)); dy ~ N(0, 1).
* ``c3``  one layer 1024 -> 1024, batch 8192, float32, G in {8, 20, 50}, no
  base branch (the grid sizes of the InKAN "Performance" table);
  x ~ U(-1, 1); C ~ N(0, 0.05); dy ~ N(0, 1).
* ``c4``  two layers 768 -> 3072 -> 768, 12608 rows (64 images x 197
  tokens), G = 5, bf16 x / C / W_base, base branch (the ViT-style channel
  mixer of the Kolmogorov-Arnold Transformer that FlashKAT studies);
  x ~ N(0, 0.3) clamped; C ~ N(0, 0.02); W_base ~ N(0, 1/sqrt(in));
  dy ~ N(0, 1).  The hidden activation is rounded to bf16 between layers.
* ``c5``  one layer 4096 -> 4096, 65536 rows, G = 20, bf16 x / C / W_base,
  base branch; x ~ U(-1, 1); C ~ N(0, 0.02); W_base ~ N(0, 1/64);
  dy ~ N(0, 1).

Grouped spline activation workloads (``make_grouped``):

* ``g1``  25216 rows (128 images x 197 tokens) by 3072 channels (the hidden
  width of a ViT-B channel mixer), 8 groups of 384 channels, G = 5, bf16 x
  and C: the shape of the grouped KAN activations of the Kolmogorov-Arnold
  Transformer that FlashKAT studies; x ~ U(-1, 1); C ~ N(0, 0.3);
  dy ~ N(0, 1).
* ``g2``  32768 rows (8 sequences x 4096 tokens) by 2048 channels, one
  spline per channel (2048 groups), G = 8, bf16 x and C: per-coordinate
  spline curves over a 2048-wide projection; same draws.

2-D tensor-product layer workload (``make_surface``):

* ``s1``  8192 rows, 1024 inputs taken as 512 consecutive pairs -> 1024
  outputs, G = 5, bf16 x and C (the 1024 -> 1024 layer of the InKAN
  performance table, with bicubic surfaces over input pairs);
  x ~ U(-1, 1); C ~ N(0, 0.02); dy ~ N(0, 1).

``N(0, s)`` means standard deviation ``s``.  Draws are float32 from NumPy's
``default_rng`` seeded by ``SeedSequence([1000 + id, G])``, with child
streams spawned in the order x, then per layer C and W_base, then dy.  bf16
tensors are float32 draws rounded to nearest-even by torch's CPU cast and
kept as float32 arrays whose values are exactly representable in bf16.
"""

import math

import numpy as np

CONFIGS = {
    "c1": dict(id=1, N=32, widths=[8, 4], G=8, lo=-1.0, hi=1.0, dtype="f32",
               base=False, x=("uniform", 1.0), clamp=True, c_std=0.1),
    "c2": dict(id=2, N=1024, widths=[784, 64, 10], G=8, lo=-1.0, hi=1.0, dtype="f32",
               base=True, x=("normal", 0.5), clamp=True, c_std=0.1),
    "c3": dict(id=3, N=8192, widths=[1024, 1024], G=8, lo=-1.0, hi=1.0, dtype="f32",
               base=False, x=("uniform", 1.0), clamp=False, c_std=0.05,
               grids=(8, 20, 50)),
    "c4": dict(id=4, N=12608, widths=[768, 3072, 768], G=5, lo=-1.0, hi=1.0, dtype="bf16",
               base=True, x=("normal", 0.3), clamp=True, c_std=0.02),
    "c5": dict(id=5, N=65536, widths=[4096, 4096], G=20, lo=-1.0, hi=1.0, dtype="bf16",
               base=True, x=("uniform", 1.0), clamp=False, c_std=0.02),
}


GROUPED = {
    "g1": dict(id=11, N=25216, I=3072, groups=8, G=5, lo=-1.0, hi=1.0, dtype="bf16"),
    "g2": dict(id=12, N=32768, I=2048, groups=2048, G=8, lo=-1.0, hi=1.0, dtype="bf16"),
}


SURFACE = {
    "s1": dict(id=21, N=8192, P=512, O=1024, G=5, lo=-1.0, hi=1.0, dtype="bf16", c_std=0.02),
}


def to_bf16_values(a):
    """float32 array -> float32 array holding the nearest-even bf16 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _draw_x(rng, shape, kind, clamp):
    dist, s = kind
    if dist == "uniform":
        x = (rng.random(shape, dtype=np.float32) * np.float32(2 * s) - np.float32(s))
    else:
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(s)
    if clamp:
        np.clip(x, -1.0, 1.0, out=x)
    return x


def make_workload(name, G=None, N=None, degree=3):
    """Inputs of one workload as a dict of NumPy float32 arrays.

    Keys: ``name, N, widths, G, lo, hi, dtype, base, x, layers`` (list of
    ``(C [O, I, G+3], W [O, I] or None)``) and ``dy [N, O_last]``.  ``G``
    selects the grid for ``c3``; ``N`` may shrink the batch (the first ``N``
    rows are drawn from the same streams, for quick tests).  ``degree`` other
    than 3 gives ``C [O, I, G + degree]`` from the same streams.
    """
    spec = dict(CONFIGS[name])
    if G is None:
        G = spec["G"]
    spec["G"] = G
    Nfull = spec["N"]
    N = Nfull if N is None else N
    widths = spec["widths"]
    nl = len(widths) - 1
    ss = np.random.SeedSequence([1000 + spec["id"], G])
    kids = ss.spawn(1 + 2 * nl + 1)
    bf16 = spec["dtype"] == "bf16"
    x = _draw_x(np.random.default_rng(kids[0]), (N, widths[0]), spec["x"], spec["clamp"])
    if bf16:
        x = to_bf16_values(x)
    layers = []
    for l in range(nl):
        I, O = widths[l], widths[l + 1]
        C = np.random.default_rng(kids[1 + 2 * l]).standard_normal(
            (O, I, G + degree), dtype=np.float32) * np.float32(spec["c_std"])
        W = None
        if spec["base"]:
            W = np.random.default_rng(kids[2 + 2 * l]).standard_normal(
                (O, I), dtype=np.float32) * np.float32(1.0 / math.sqrt(I))
        if bf16:
            C = to_bf16_values(C)
            W = None if W is None else to_bf16_values(W)
        layers.append((C, W))
    dy = np.random.default_rng(kids[-1]).standard_normal((N, widths[-1]), dtype=np.float32)
    return dict(name=name, N=N, widths=list(widths), G=G, lo=spec["lo"], hi=spec["hi"],
                dtype=spec["dtype"], base=spec["base"], x=x, layers=layers, dy=dy)


def random_layer(N, I, O, G, dtype="f32", base=True, seed=0, lo=-1.0, hi=1.0,
                 x_scale=1.0, special=True, degree=3):
    """A small random layer for parity tests.

    ``x`` is drawn ~U(-x_scale, x_scale) * (hi - lo) / 2 around the grid
    centre.  With ``special`` a share of the entries is replaced by points
    the span logic must get right: every knot of the extended grid, ``lo``,
    ``hi``, points just inside/outside them, and points far outside the
    extended grid.  ``degree`` other than 3 draws ``C [O, I, G + degree]`` and
    takes the knots of that grid (extended by ``degree`` per side).
    """
    seq = [7, seed, N, I, O, G] + ([] if degree == 3 else [degree])
    rng = np.random.default_rng(np.random.SeedSequence(seq))
    mid, half = 0.5 * (lo + hi), 0.5 * (hi - lo)
    x = (mid + half * x_scale * (2 * rng.random((N, I)) - 1)).astype(np.float32)
    if special and N * I > 0:
        h = (hi - lo) / G
        pts = [lo + (r - degree) * h for r in range(G + 2 * degree + 1)]
        pts += [lo, hi, np.nextafter(np.float32(hi), np.float32(-np.inf)),
                np.nextafter(np.float32(hi), np.float32(np.inf)),
                np.nextafter(np.float32(lo), np.float32(-np.inf)),
                lo - degree * h - 1e-3, hi + degree * h + 1e-3, lo - 10.0, hi + 10.0, 0.0]
        pts = np.asarray(pts, dtype=np.float32)
        mask = rng.random((N, I)) < 0.25
        x[mask] = pts[rng.integers(0, len(pts), size=int(mask.sum()))]
    C = (rng.standard_normal((O, I, G + degree)) * 0.1).astype(np.float32)
    W = (rng.standard_normal((O, I)) / math.sqrt(I)).astype(np.float32) if base else None
    dy = rng.standard_normal((N, O)).astype(np.float32)
    if dtype == "bf16":
        x = to_bf16_values(x)
        C = to_bf16_values(C)
        W = None if W is None else to_bf16_values(W)
    return dict(N=N, widths=[I, O], G=G, lo=lo, hi=hi, dtype=dtype, base=base,
                x=x, layers=[(C, W)], dy=dy)


def sample_indices(n, count, seed):
    """``count`` distinct sorted indices in ``[0, n)`` (all of them if ``count >= n``)."""
    if count >= n:
        return np.arange(n)
    rng = np.random.default_rng(np.random.SeedSequence([4242, seed, n]))
    return np.sort(rng.choice(n, size=count, replace=False))


def sample_pairs(O, I, count, seed):
    """``count`` seeded ``(j, i)`` pairs, ``j < O``, ``i < I``."""
    rng = np.random.default_rng(np.random.SeedSequence([4343, seed, O, I]))
    js = rng.integers(0, O, size=count)
    is_ = rng.integers(0, I, size=count)
    return np.stack([js, is_], axis=1)


def make_grouped(name, N=None):
    """Inputs of one grouped activation workload: dict with ``name, N, I,
    groups, G, lo, hi, dtype, x [N, I], C [groups, G+3], dy [N, I]`` (float32
    arrays; bf16 workloads hold bf16-exact values).  ``N`` may shrink the
    batch (the first rows of the same streams)."""
    spec = dict(GROUPED[name])
    Nfull, I, groups, G = spec["N"], spec["I"], spec["groups"], spec["G"]
    N = Nfull if N is None else N
    kids = np.random.SeedSequence([1000 + spec["id"], G]).spawn(3)
    x = _draw_x(np.random.default_rng(kids[0]), (N, I), ("uniform", 1.0), False)
    C = np.random.default_rng(kids[1]).standard_normal((groups, G + 3), dtype=np.float32) * np.float32(0.3)
    dy = np.random.default_rng(kids[2]).standard_normal((N, I), dtype=np.float32)
    if spec["dtype"] == "bf16":
        x = to_bf16_values(x)
        C = to_bf16_values(C)
    spec.update(name=name, N=N, x=x, C=C, dy=dy)
    return spec


def random_grouped(N, I, groups, G, dtype="f32", seed=0, lo=-1.0, hi=1.0, special=True):
    """A small random grouped activation for parity tests; ``special`` mixes in
    the knots and the points around and far outside the grid, as
    ``random_layer`` does."""
    rng = np.random.default_rng(np.random.SeedSequence([9, seed, N, I, groups, G]))
    mid, half = 0.5 * (lo + hi), 0.5 * (hi - lo)
    x = (mid + half * 1.3 * (2 * rng.random((N, I)) - 1)).astype(np.float32)
    if special and N * I > 0:
        h = (hi - lo) / G
        pts = [lo + (r - 3) * h for r in range(G + 7)]
        pts += [lo, hi, np.nextafter(np.float32(hi), np.float32(-np.inf)),
                np.nextafter(np.float32(lo), np.float32(-np.inf)),
                lo - 3 * h - 1e-3, hi + 3 * h + 1e-3, lo - 10.0, hi + 10.0, 0.0]
        pts = np.asarray(pts, dtype=np.float32)
        mask = rng.random((N, I)) < 0.25
        x[mask] = pts[rng.integers(0, len(pts), size=int(mask.sum()))]
    C = (rng.standard_normal((groups, G + 3)) * 0.3).astype(np.float32)
    dy = rng.standard_normal((N, I)).astype(np.float32)
    if dtype == "bf16":
        x = to_bf16_values(x)
        C = to_bf16_values(C)
    return dict(N=N, I=I, groups=groups, G=G, lo=lo, hi=hi, dtype=dtype, x=x, C=C, dy=dy)


def make_surface(name, N=None):
    """Inputs of a 2-D layer workload: dict with ``name, N, P, O, G, lo, hi,
    dtype, x [N, 2P], C [O, P, G+3, G+3], dy [N, O]``."""
    spec = dict(SURFACE[name])
    P, O, G = spec["P"], spec["O"], spec["G"]
    N = spec["N"] if N is None else N
    kids = np.random.SeedSequence([1000 + spec["id"], G]).spawn(3)
    x = _draw_x(np.random.default_rng(kids[0]), (N, 2 * P), ("uniform", 1.0), False)
    C = np.random.default_rng(kids[1]).standard_normal((O, P, G + 3, G + 3), dtype=np.float32) \
        * np.float32(spec["c_std"])
    dy = np.random.default_rng(kids[2]).standard_normal((N, O), dtype=np.float32)
    if spec["dtype"] == "bf16":
        x = to_bf16_values(x)
        C = to_bf16_values(C)
    spec.update(name=name, N=N, x=x, C=C, dy=dy)
    return spec


def random_surface(N, P, O, G, dtype="f32", seed=0, lo=-1.0, hi=1.0, special=True):
    """A small random 2-D layer for parity tests (x mixed with the knots and
    points around and far outside the grid, as in ``random_layer``)."""
    rng = np.random.default_rng(np.random.SeedSequence([11, seed, N, P, O, G]))
    mid, half = 0.5 * (lo + hi), 0.5 * (hi - lo)
    x = (mid + half * 1.2 * (2 * rng.random((N, 2 * P)) - 1)).astype(np.float32)
    if special and N * P > 0:
        h = (hi - lo) / G
        pts = [lo + (r - 3) * h for r in range(G + 7)]
        pts += [lo, hi, np.nextafter(np.float32(hi), np.float32(-np.inf)),
                lo - 3 * h - 1e-3, hi + 3 * h + 1e-3, lo - 10.0, hi + 10.0, 0.0]
        pts = np.asarray(pts, dtype=np.float32)
        mask = rng.random((N, 2 * P)) < 0.2
        x[mask] = pts[rng.integers(0, len(pts), size=int(mask.sum()))]
    C = (rng.standard_normal((O, P, G + 3, G + 3)) * 0.1).astype(np.float32)
    dy = rng.standard_normal((N, O)).astype(np.float32)
    if dtype == "bf16":
        x = to_bf16_values(x)
        C = to_bf16_values(C)
    return dict(N=N, P=P, O=O, G=G, lo=lo, hi=hi, dtype=dtype, x=x, C=C, dy=dy)
