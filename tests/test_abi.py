"""C ABI checks that need no GPU: the library loads, exports every symbol
``include/kan.h`` declares, and returns each validation error before any
device work (pointers here are fake addresses that are never dereferenced)."""

import ctypes
import os
import re
import subprocess

import pytest

from kan_testutil import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kan.h")


@pytest.fixture(scope="module")
def L():
    ensure_built()
    from kolmogorov_arnold_network_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kan_\w+)\s*\(", src, flags=re.M)))


def test_header_lists_the_binding_exports():
    assert declared_functions() == sorted(
        __import__("kolmogorov_arnold_network_amd._lib", fromlist=["EXPORTS"]).EXPORTS)


def test_every_declared_symbol_is_exported(L):
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    from kolmogorov_arnold_network_amd._build import LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_version_and_status_strings(L):
    assert L.lib().kan_abi_version() == L.ABI_VERSION == 1
    for code in range(0, -10, -1):
        s = L.status_string(code)
        assert s and s != "unknown status"
    assert L.status_string(42) == "unknown status"


def test_struct_layout(L):
    assert ctypes.sizeof(L.kan_grid_t) == 16
    assert ctypes.sizeof(L.kan_desc_t) == 3 * 8 + 16 + 4 * 4


# fake, 256-aligned, non-overlapping device addresses (never dereferenced)
X, C, W, Y, WS, DY, DX, DC, DW = [0x100000000 * (k + 1) for k in range(9)]


def desc(L, **kw):
    a = dict(N=64, I=16, O=8, lo=-1.0, hi=1.0, G=8, dtype=L.KAN_F32, has_base=1,
             variant=L.KAN_VARIANT_MFMA, flags=0)
    a.update(kw)
    return L.make_desc(**a)


def fwd(L, d, x=X, c=C, w=W, y=Y, ws=WS, nbytes=None):
    if nbytes is None:
        nbytes = L.lib().kan_workspace_size(ctypes.byref(d), L.KAN_PASS_FORWARD)
    return L.lib().kan_forward(ctypes.byref(d), x, c, w, y, ws, nbytes, None)


def bwd(L, d, x=X, c=C, w=W, dy=DY, dx=DX, dc=DC, dw=DW, ws=WS, nbytes=None):
    if nbytes is None:
        nbytes = L.lib().kan_workspace_size(ctypes.byref(d), L.KAN_PASS_BACKWARD)
    return L.lib().kan_backward(ctypes.byref(d), x, c, w, dy, dx, dc, dw, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), "SHAPE"), (dict(I=0), "SHAPE"), (dict(O=0), "SHAPE"), (dict(N=1 << 40), "SHAPE"),
    (dict(G=0), "GRID"), (dict(G=126), "GRID"), (dict(G=5000), "GRID"), (dict(lo=1.0, hi=1.0), "GRID"),
    (dict(lo=2.0, hi=1.0), "GRID"), (dict(lo=float("nan")), "GRID"), (dict(hi=float("inf")), "GRID"),
    (dict(degree=0), "UNSUPPORTED"), (dict(degree=6), "UNSUPPORTED"),
    (dict(degree=2, variant=2), "UNSUPPORTED"),                 # degree != 3: matrix cores only
    (dict(degree=1, G=1, has_base=0), "UNSUPPORTED"),           # 2 columns per input: too few
    (dict(dtype=7), "DTYPE"), (dict(has_base=2), "UNSUPPORTED"),
    (dict(variant=9), "UNSUPPORTED"), (dict(flags=4), "UNSUPPORTED"),
])
def test_bad_descriptors(L, kw, code):
    d = desc(L, **kw)
    want = getattr(L, "KAN_ERR_" + code)
    assert fwd(L, d, nbytes=1 << 40) == want
    assert bwd(L, d, nbytes=1 << 40) == want
    assert L.lib().kan_workspace_size(ctypes.byref(d), 0) == ctypes.c_size_t(-1).value


def test_null_desc(L):
    lib = L.lib()
    assert lib.kan_forward(None, X, C, W, Y, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_backward(None, X, C, W, DY, DX, DC, DW, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_workspace_size(None, 0) == ctypes.c_size_t(-1).value


def test_forward_pointer_checks(L):
    d = desc(L)
    assert fwd(L, d, x=None) == L.KAN_ERR_NULL
    assert fwd(L, d, y=None) == L.KAN_ERR_NULL
    assert fwd(L, d, c=None) == L.KAN_ERR_NULL
    assert fwd(L, d, w=None) == L.KAN_ERR_NULL                     # has_base=1 needs W
    assert fwd(L, desc(L, has_base=0)) == L.KAN_ERR_NULL          # has_base=0 forbids W
    assert fwd(L, d, x=X + 8) == L.KAN_ERR_ALIGN
    assert fwd(L, d, y=Y + 4) == L.KAN_ERR_ALIGN
    assert fwd(L, d, ws=WS + 128) == L.KAN_ERR_ALIGN
    assert fwd(L, d, nbytes=16) == L.KAN_ERR_WORKSPACE
    assert fwd(L, d, ws=None) == L.KAN_ERR_NULL
    assert fwd(L, d, y=X + 64) == L.KAN_ERR_ALIAS
    assert fwd(L, d, y=C) == L.KAN_ERR_ALIAS
    assert fwd(L, d, ws=Y) == L.KAN_ERR_ALIAS


def test_backward_pointer_checks(L):
    d = desc(L)
    assert bwd(L, d, dy=None) == L.KAN_ERR_NULL
    assert bwd(L, d, x=None) == L.KAN_ERR_NULL
    assert bwd(L, desc(L, has_base=0), w=None) == L.KAN_ERR_NULL  # dW given without base
    assert bwd(L, d, dy=DY + 2) == L.KAN_ERR_ALIGN
    assert bwd(L, d, dc=DC + 4) == L.KAN_ERR_ALIGN
    assert bwd(L, d, nbytes=0) == L.KAN_ERR_WORKSPACE
    assert bwd(L, d, dx=DC) == L.KAN_ERR_ALIAS
    assert bwd(L, d, dw=DY) == L.KAN_ERR_ALIAS
    assert bwd(L, d, dc=X) == L.KAN_ERR_ALIAS
    assert bwd(L, d, ws=DX) == L.KAN_ERR_ALIAS


def test_empty_batch_forward_returns_ok_without_launch(L):
    assert fwd(L, desc(L, N=0)) == L.KAN_OK


def k_slices(tiles, nkt, out_bytes, esize):
    """The planner's k-split rule, restated: slices of the k range for a
    contraction of `tiles` output tiles over `nkt` k-tiles with `out_bytes`
    of fp32 output (estimate: rounds of 256 one-per-CU workgroups x k-tiles
    per workgroup at 2 us (bf16) or 8 us (fp32), plus 2P + 1 passes over
    the partials at 4 bytes/ns; taken when it saves >= 1/16, >= 8 k-tiles a
    slice).  Returns (slices, k-tiles per slice)."""
    kt_ns = 2000 if esize == 2 else 8000

    def est(P):
        per, rounds = (nkt + P - 1) // P, (tiles * P + 255) // 256
        return rounds * per * kt_ns + ((2 * P + 1) * out_bytes // 4000 if P > 1 else 0)
    best, tb = 1, est(1)
    P = 2
    while P <= 8 and (nkt + P - 1) // P >= 8:
        if est(P) < tb:
            best, tb = P, est(P)
        P += 1
    if tb > est(1) - est(1) // 16:
        best = 1
    nks = (nkt + best - 1) // best
    return (nkt + nks - 1) // nks, nks


def test_workspace_sizes(L):
    ws = lambda **kw: L.lib().kan_workspace_size(ctypes.byref(desc(L, **kw)), 0)
    wb = lambda **kw: L.lib().kan_workspace_size(ctypes.byref(desc(L, **kw)), 1)
    assert ws(variant=L.KAN_VARIANT_GATHER) == 0 and wb(variant=L.KAN_VARIANT_GATHER) == 0
    # MFMA forward: packed C' [O padded to 256][I*Kb padded to the k-tile]
    r = lambda a, b: (a + b - 1) // b * b
    for dt, es, bk in [(L.KAN_F32, 4, 32), (L.KAN_BF16, 2, 64)]:
        for (N, I, O, G, base) in [(64, 16, 8, 8, 1), (1000, 777, 300, 20, 0), (5, 3, 2, 1, 1),
                                   (12608, 768, 3072, 5, 1), (12608, 3072, 768, 5, 1), (8192, 1024, 1024, 50, 0)]:
            Kb = G + 3 + base
            # bf16 forwards with 11 <= Kb <= 32 whose 2:4 layout (NG groups of 4
            # columns per input) costs <= 3/4 of the dense one pack I * 4 NG columns
            ng = max(4, (Kb + 3) // 4)
            ng += ng & 1
            sparse = dt == L.KAN_BF16 and ng <= 8 and Kb >= 11 and 8 * ng <= 3 * Kb
            Op, Np = r(O, 256), r(N, 256)

            def fwd_bytes(kf, nkt):
                # packed C', then the partial y of a split forward
                P, _ = k_slices((Np // 256) * (Op // 256), nkt, N * O * 4, es)
                return r(Op * kf * es, 256) + (r(P * N * O * 4, 256) if P > 1 else 0)
            kf = r(I * 4 * ng, 64) if sparse else r(I * Kb, bk)
            assert ws(N=N, I=I, O=O, G=G, has_base=base, dtype=dt) == fwd_bytes(kf, kf // (64 if sparse else bk))
            if sparse:
                assert L.lib().kan_workspace_size(ctypes.byref(desc(
                    L, N=N, I=I, O=O, G=G, has_base=base, dtype=dt, flags=L.KAN_FLAG_DENSE_FORWARD)), 0) == \
                    fwd_bytes(r(I * Kb, bk), r(I * Kb, bk) // bk)
            tiles = (I * Kb + 255) // 256           # dx tiles of 256 P columns
            want = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 2 * 4, 256)
            P, _ = k_slices((Op // 256) * tiles, Np // bk, O * I * Kb * 4, es)   # dC over batch slices
            want += r(P * O * I * Kb * 4, 256) if P > 1 else 0
            assert wb(N=N, I=I, O=O, G=G, has_base=base, dtype=dt) == want
    # auto: bf16 on the matrix cores; float32 forward on the gather kernel and
    # backward on the matrix cores
    assert ws(G=125, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) > 0      # largest grid: MFMA fits
    assert ws(G=126, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) == ctypes.c_size_t(-1).value
    # float32 AUTO: gather forward (no workspace), matrix-core backward
    assert ws(variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_F32) == 0
    assert wb(N=64, I=32, O=32, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_F32) == wb(
        N=64, I=32, O=32, variant=L.KAN_VARIANT_MFMA, dtype=L.KAN_F32) > 0          # 2^16 edge-rows
    assert wb(N=63, I=32, O=32, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_F32) == 0  # below: gather
    assert ws(variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) == ws(variant=L.KAN_VARIANT_MFMA,
                                                                   dtype=L.KAN_BF16) > 0


def test_workspace_sizes_other_degrees(L):
    """Degree D != 3: K = G + D columns per input, both passes on the matrix
    cores whatever the variant asked (AUTO), never the structured-sparse
    forward, otherwise the cubic layout."""
    r = lambda a, b: (a + b - 1) // b * b
    for dt, es, bk in [(L.KAN_F32, 4, 32), (L.KAN_BF16, 2, 64)]:
        for (N, I, O, G, base, D) in [(64, 16, 8, 8, 1, 1), (1000, 77, 300, 20, 0, 5), (12608, 768, 3072, 5, 1, 2),
                                      (5, 3, 2, 1, 1, 4)]:
            Kb = G + D + base
            Op, Np = r(O, 256), r(N, 256)
            kf = r(I * Kb, bk)
            P, _ = k_slices((Np // 256) * (Op // 256), kf // bk, N * O * 4, es)
            want_f = r(Op * kf * es, 256) + (r(P * N * O * 4, 256) if P > 1 else 0)
            tiles = (I * Kb + 255) // 256
            want_b = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 2 * 4, 256)
            Pd, _ = k_slices((Op // 256) * tiles, Np // bk, O * I * Kb * 4, es)
            want_b += r(Pd * O * I * Kb * 4, 256) if Pd > 1 else 0
            d = desc(L, N=N, I=I, O=O, G=G, has_base=base, dtype=dt, degree=D, variant=L.KAN_VARIANT_AUTO)
            assert L.lib().kan_workspace_size(ctypes.byref(d), 0) == want_f
            assert L.lib().kan_workspace_size(ctypes.byref(d), 1) == want_b


def test_prepare_checks(L):
    d = desc(L)
    lib = L.lib()
    assert lib.kan_prepare(ctypes.byref(d), 5, C, W, DY, WS, 1 << 30, None) == L.KAN_ERR_UNSUPPORTED
    assert lib.kan_prepare(ctypes.byref(d), 0, None, W, None, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_prepare(ctypes.byref(d), 1, C, W, None, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_prepare(ctypes.byref(d), 0, C, W, None, C, 1 << 30, None) == L.KAN_ERR_ALIAS


@pytest.mark.parametrize("fn", ["kan_basis_eval", "kan_basis_eval_tp"])
def test_basis_checks(L, fn):
    f = getattr(L.lib(), fn)
    g = L.kan_grid_t(-1.0, 1.0, 8, 3)
    assert f(None, 4, 0, X, Y, DY, None) == L.KAN_ERR_NULL
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 0, 3)), 4, 0, X, Y, None, None) == L.KAN_ERR_GRID
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 126, 3)), 4, 0, X, Y, None, None) == L.KAN_ERR_GRID
    # the basis step takes degrees 1 .. 5 (the layer only 3)
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 8, 0)), 4, 0, X, Y, None, None) == L.KAN_ERR_UNSUPPORTED
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 8, 6)), 4, 0, X, Y, None, None) == L.KAN_ERR_UNSUPPORTED
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 8, 5)), 0, 0, X, Y, None, None) == L.KAN_OK
    assert f(ctypes.byref(L.kan_grid_t(-1.0, 1.0, 8, 5)), 4, 0, X, X - 64, None, None) == L.KAN_ERR_ALIAS
    assert f(ctypes.byref(g), -1, 0, X, Y, None, None) == L.KAN_ERR_SHAPE
    assert f(ctypes.byref(g), 0, 0, X, Y, None, None) == L.KAN_OK
    assert f(ctypes.byref(g), 4, 0, X, None, None, None) == L.KAN_ERR_NULL
    assert f(ctypes.byref(g), 4, 3, X, Y, None, None) == L.KAN_ERR_DTYPE
    assert f(ctypes.byref(g), 4, 0, X + 4, Y, None, None) == L.KAN_ERR_ALIGN
    assert f(ctypes.byref(g), 4, 0, X, X, None, None) == L.KAN_ERR_ALIAS


def test_cast_checks(L):
    lib = L.lib()
    assert lib.kan_cast_f32_to_bf16(X, Y, -1, None) == L.KAN_ERR_SHAPE
    assert lib.kan_cast_f32_to_bf16(X, Y, 0, None) == L.KAN_OK
    assert lib.kan_cast_f32_to_bf16(None, Y, 4, None) == L.KAN_ERR_NULL
    assert lib.kan_cast_f32_to_bf16(X + 2, Y, 4, None) == L.KAN_ERR_ALIGN
    assert lib.kan_cast_f32_to_bf16(X, X + 16, 8, None) == L.KAN_ERR_ALIAS


def gdesc(L, N=100, I=300, groups=5, G=8, dtype=0, lo=-1.0, hi=1.0, degree=3):
    return L.make_group_desc(N, I, groups, lo, hi, G, dtype, degree)


def group_workspace(N, I, K):
    """The grouped backward's workspace, restated: channel blocks of 64, row
    chunks aimed at no more than 1024 blocks, with at least max(64, 24 K) rows
    (a multiple of 32: 4 row waves of 8 rows), K floats per channel per chunk,
    then K per channel summed."""
    if N == 0:
        return 0
    xb = (I + 63) // 64
    gy = max(1, 1024 // xb)
    R = max(max(64, 24 * K), (N + gy - 1) // gy)
    R = (R + 31) // 32 * 32
    chunks = (N + R - 1) // R
    return ((chunks * K * I + K * I) * 4 + 255) // 256 * 256


def test_group_struct_layout(L):
    assert ctypes.sizeof(L.kan_group_desc_t) == 2 * 8 + 2 * 4 + 16


def test_group_workspace_sizes(L):
    f = lambda d: L.lib().kan_group_workspace_size(ctypes.byref(d))
    for (N, I, groups, G) in [(100, 300, 5, 8), (25216, 3072, 8, 5), (32768, 2048, 2048, 8),
                              (1, 1, 1, 1), (1000000, 17, 17, 125), (0, 5, 5, 3)]:
        assert f(gdesc(L, N=N, I=I, groups=groups, G=G)) == group_workspace(N, I, G + 3)
        assert f(gdesc(L, N=N, I=I, groups=groups, G=G, dtype=1)) == group_workspace(N, I, G + 3)
    bad = ctypes.c_size_t(-1).value
    assert L.lib().kan_group_workspace_size(None) == bad
    assert f(gdesc(L, groups=301)) == bad
    assert f(gdesc(L, G=126)) == bad
    assert f(gdesc(L, N=10, I=(1 << 31) // 11, groups=1, G=8)) == bad     # I * (G+3) beyond the index range


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), -2), (dict(I=0), -2), (dict(groups=0), -2), (dict(groups=301), -2),
    (dict(N=1 << 40), -2), (dict(G=0), -3), (dict(G=126), -3), (dict(lo=1.0, hi=1.0), -3),
    (dict(lo=float("nan")), -3), (dict(dtype=2), -4), (dict(degree=2), -8)])
def test_group_bad_descriptors(L, kw, code):
    d = gdesc(L, **kw)
    lib = L.lib()
    assert lib.kan_group_forward(ctypes.byref(d), X, C, Y, None) == code
    assert lib.kan_group_backward(ctypes.byref(d), X, C, DY, DX, DC, WS, 1 << 30, None) == code


def test_group_pointer_checks(L):
    d = gdesc(L)
    lib = L.lib()
    n = lib.kan_group_workspace_size(ctypes.byref(d))
    fwd = lambda *a: lib.kan_group_forward(ctypes.byref(d), *a, None)
    bwd = lambda *a: lib.kan_group_backward(ctypes.byref(d), *a, None)
    assert lib.kan_group_forward(None, X, C, Y, None) == L.KAN_ERR_NULL
    assert fwd(None, C, Y) == L.KAN_ERR_NULL
    assert fwd(X, None, Y) == L.KAN_ERR_NULL
    assert fwd(X, C, None) == L.KAN_ERR_NULL
    assert fwd(X + 8, C, Y) == L.KAN_ERR_ALIGN
    assert fwd(X, C, X + 16) == L.KAN_ERR_ALIAS                 # y over x
    assert fwd(X, C, C) == L.KAN_ERR_ALIAS                      # y over C
    assert bwd(None, C, DY, DX, DC, WS, n) == L.KAN_ERR_NULL
    assert bwd(X, C, None, DX, DC, WS, n) == L.KAN_ERR_NULL
    assert bwd(X, C, DY, DX, DC, WS, n - 1) == L.KAN_ERR_WORKSPACE
    assert bwd(X, C, DY, DX, DC, None, n) == L.KAN_ERR_NULL
    assert bwd(X, C, DY, DX, DC, WS + 16, n) == L.KAN_ERR_ALIGN
    assert bwd(X, C, DY, DX + 4, DC, WS, n) == L.KAN_ERR_ALIGN
    assert bwd(X, C, DY, DY, DC, WS, n) == L.KAN_ERR_ALIAS      # dx over dy
    assert bwd(X, C, DY, DX, DX, WS, n) == L.KAN_ERR_ALIAS      # dC over dx
    assert bwd(X, C, DY, DX, DC, DC, n) == L.KAN_ERR_ALIAS      # workspace over dC
    assert bwd(X, C, DY, None, None, None, 0) == L.KAN_OK       # nothing asked: no work
    e = gdesc(L, N=0)
    assert lib.kan_group_forward(ctypes.byref(e), None, C, None, None) == L.KAN_OK


def sdesc(L, N=100, P=8, O=20, G=5, dtype=1, lo=-1.0, hi=1.0, degree=3, flags=0):
    return L.make_surface_desc(N, P, O, lo, hi, G, dtype, degree, flags)


def test_surface_struct_layout(L):
    assert ctypes.sizeof(L.kan_surface_desc_t) == 3 * 8 + 16 + 2 * 4


def test_surface_workspace_sizes(L):
    """The layer's layout restated for pairs: K = Kb = (G+3)^2 columns per
    pair, no structured-sparse forward, and dx partials for both inputs of a
    pair cut by a tile edge."""
    r = lambda a, b: (a + b - 1) // b * b
    for dt, es, bk in [(0, 4, 32), (1, 2, 64)]:
        for (N, P, O, G) in [(100, 8, 20, 5), (8192, 512, 1024, 5), (300, 7, 33, 8), (5, 3, 2, 1),
                             (77, 4, 300, 13)]:
            Kb = (G + 3) ** 2
            Op, Np = r(O, 256), r(N, 256)
            kf = r(P * Kb, bk)
            Pf, _ = k_slices((Np // 256) * (Op // 256), kf // bk, N * O * 4, es)
            want_f = r(Op * kf * es, 256) + (r(Pf * N * O * 4, 256) if Pf > 1 else 0)
            tiles = (P * Kb + 255) // 256
            want_b = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 4 * 4, 256)
            Pd, _ = k_slices((Op // 256) * tiles, Np // bk, O * P * Kb * 4, es)
            want_b += r(Pd * O * P * Kb * 4, 256) if Pd > 1 else 0
            d = sdesc(L, N=N, P=P, O=O, G=G, dtype=dt)
            assert L.lib().kan_surface_workspace_size(ctypes.byref(d), 0) == want_f
            assert L.lib().kan_surface_workspace_size(ctypes.byref(d), 1) == want_b
    bad = ctypes.c_size_t(-1).value
    assert L.lib().kan_surface_workspace_size(ctypes.byref(sdesc(L)), 2) == bad
    assert L.lib().kan_surface_workspace_size(None, 0) == bad


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), -2), (dict(P=0), -2), (dict(O=0), -2), (dict(G=0), -3), (dict(G=14), -3),
    (dict(lo=1.0, hi=0.5), -3), (dict(hi=float("inf")), -3), (dict(dtype=5), -4), (dict(degree=1), -8),
    (dict(flags=4), -8), (dict(P=1 << 30), -2)])
def test_surface_bad_descriptors(L, kw, code):
    d = sdesc(L, **kw)
    lib = L.lib()
    assert lib.kan_surface_forward(ctypes.byref(d), X, C, Y, WS, 1 << 40, None) == code
    assert lib.kan_surface_backward(ctypes.byref(d), X, C, DY, DX, DC, WS, 1 << 40, None) == code


def test_surface_pointer_checks(L):
    d = sdesc(L)
    lib = L.lib()
    nf = lib.kan_surface_workspace_size(ctypes.byref(d), 0)
    nb = lib.kan_surface_workspace_size(ctypes.byref(d), 1)
    fwd = lambda *a: lib.kan_surface_forward(ctypes.byref(d), *a, None)
    bwd = lambda *a: lib.kan_surface_backward(ctypes.byref(d), *a, None)
    assert fwd(None, C, Y, WS, nf) == L.KAN_ERR_NULL
    assert fwd(X, None, Y, WS, nf) == L.KAN_ERR_NULL
    assert fwd(X, C, None, WS, nf) == L.KAN_ERR_NULL
    assert fwd(X + 2, C, Y, WS, nf) == L.KAN_ERR_ALIGN
    assert fwd(X, C, Y, WS, nf - 1) == L.KAN_ERR_WORKSPACE
    assert fwd(X, C, Y, WS + 64, nf) == L.KAN_ERR_ALIGN
    assert fwd(X, C, X, WS, nf) == L.KAN_ERR_ALIAS
    assert fwd(X, C, Y, C, nf) == L.KAN_ERR_ALIAS
    assert bwd(X, C, None, DX, DC, WS, nb) == L.KAN_ERR_NULL
    assert bwd(X, C, DY, DX, DC, WS, nb - 1) == L.KAN_ERR_WORKSPACE
    assert bwd(X, C, DY, DY, DC, WS, nb) == L.KAN_ERR_ALIAS
    assert bwd(X, C, DY, DX, DX, WS, nb) == L.KAN_ERR_ALIAS
    assert bwd(X, C, DY, None, None, WS, nb) == L.KAN_OK        # nothing asked: no work


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from kolmogorov_arnold_network_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
