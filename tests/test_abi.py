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


# Layer descriptors every entry point must reject, with the status.  Also
# the cases tests/test_host_sanitize.py runs through the sanitizer build.
BAD_DESCS = [
    (dict(N=-1), "SHAPE"), (dict(I=0), "SHAPE"), (dict(O=0), "SHAPE"), (dict(N=1 << 40), "SHAPE"),
    (dict(G=0), "GRID"), (dict(G=126), "GRID"), (dict(G=5000), "GRID"), (dict(lo=1.0, hi=1.0), "GRID"),
    (dict(lo=2.0, hi=1.0), "GRID"), (dict(lo=float("nan")), "GRID"), (dict(hi=float("inf")), "GRID"),
    (dict(degree=0), "UNSUPPORTED"), (dict(degree=6), "UNSUPPORTED"),
    (dict(degree=1, G=1, has_base=0), "UNSUPPORTED"),           # MFMA: 2 columns per input, too few
    (dict(degree=1, G=1, has_base=0, dtype=1), "UNSUPPORTED"),  # the same in bf16
    (dict(dtype=7), "DTYPE"), (dict(has_base=2), "UNSUPPORTED"),
    (dict(variant=9), "UNSUPPORTED"), (dict(flags=8), "UNSUPPORTED"),
    # the truncated-power forward: bf16, cubic, on the matrix cores only
    (dict(flags=4), "UNSUPPORTED"), (dict(flags=4, dtype=1, degree=2), "UNSUPPORTED"),
    (dict(flags=4, dtype=1, variant=2), "UNSUPPORTED"),
]

# Pointer, alignment, workspace and overlap errors of one valid layer
# (desc() changes, call changes, status).
FWD_POINTER_CASES = [
    ({}, dict(x=None), "NULL"), ({}, dict(y=None), "NULL"), ({}, dict(c=None), "NULL"),
    ({}, dict(w=None), "NULL"),                                 # has_base=1 needs W
    (dict(has_base=0), {}, "NULL"),                             # has_base=0 forbids W
    ({}, dict(x=X + 8), "ALIGN"), ({}, dict(y=Y + 4), "ALIGN"), ({}, dict(ws=WS + 128), "ALIGN"),
    ({}, dict(nbytes=16), "WORKSPACE"), ({}, dict(ws=None), "NULL"),
    ({}, dict(y=X + 64), "ALIAS"), ({}, dict(y=C), "ALIAS"), ({}, dict(ws=Y), "ALIAS"),
]
BWD_POINTER_CASES = [
    ({}, dict(dy=None), "NULL"), ({}, dict(x=None), "NULL"),
    (dict(has_base=0), dict(w=None), "NULL"),                   # dW given without base
    ({}, dict(dy=DY + 2), "ALIGN"), ({}, dict(dc=DC + 4), "ALIGN"), ({}, dict(nbytes=0), "WORKSPACE"),
    ({}, dict(dx=DC), "ALIAS"), ({}, dict(dw=DY), "ALIAS"), ({}, dict(dc=X), "ALIAS"), ({}, dict(ws=DX), "ALIAS"),
]


@pytest.mark.parametrize("kw,code", BAD_DESCS)
def test_bad_descriptors(L, kw, code):
    d = desc(L, **kw)
    want = getattr(L, "KAN_ERR_" + code)
    assert fwd(L, d, nbytes=1 << 40) == want
    assert bwd(L, d, nbytes=1 << 40) == want
    assert L.lib().kan_workspace_size(ctypes.byref(d), 0) == ctypes.c_size_t(-1).value


def test_static_forward_checks(L):
    """kan_forward_static validates like kan_forward and, before touching
    the GPU, refuses a layer whose forward workspace exceeds its static
    array and the prepared flag (the array is shared by every call)."""
    lib = L.lib()
    stat = lambda d, **kw: lib.kan_forward_static(ctypes.byref(d), kw.get("x", X), kw.get("c", C),
                                                  kw.get("w", W), kw.get("y", Y), None)
    assert lib.kan_forward_static(None, X, C, W, Y, None) == L.KAN_ERR_NULL
    assert stat(desc(L, G=0)) == L.KAN_ERR_GRID
    assert stat(desc(L, variant=9)) == L.KAN_ERR_UNSUPPORTED
    assert stat(desc(L, flags=L.KAN_FLAG_PREPARED)) == L.KAN_ERR_UNSUPPORTED
    big = desc(L, N=65536, I=4096, O=4096, G=20, dtype=L.KAN_BF16)        # 0.8 GB of packed C'
    assert lib.kan_workspace_size(ctypes.byref(big), 0) > L.KAN_STATIC_SCRATCH_BYTES
    assert stat(big) == L.KAN_ERR_WORKSPACE
    assert stat(desc(L), w=None) == L.KAN_ERR_NULL                       # base branch needs W_base
    assert stat(desc(L), x=X + 4) == L.KAN_ERR_ALIGN
    assert stat(desc(L), y=X) == L.KAN_ERR_ALIAS
    # the quick-start layers fit the array on every variant
    for v in (L.KAN_VARIANT_AUTO, L.KAN_VARIANT_MFMA, L.KAN_VARIANT_GATHER):
        for (N, I, O) in [(1024, 784, 64), (1024, 64, 10)]:
            d = desc(L, N=N, I=I, O=O, variant=v)
            assert 0 < lib.kan_workspace_size(ctypes.byref(d), 0) <= L.KAN_STATIC_SCRATCH_BYTES


def test_null_desc(L):
    lib = L.lib()
    assert lib.kan_forward(None, X, C, W, Y, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_backward(None, X, C, W, DY, DX, DC, DW, WS, 1 << 30, None) == L.KAN_ERR_NULL
    assert lib.kan_workspace_size(None, 0) == ctypes.c_size_t(-1).value


def test_forward_pointer_checks(L):
    for dkw, ckw, code in FWD_POINTER_CASES:
        assert fwd(L, desc(L, **dkw), **ckw) == getattr(L, "KAN_ERR_" + code), (dkw, ckw)


def test_backward_pointer_checks(L):
    for dkw, ckw, code in BWD_POINTER_CASES:
        assert bwd(L, desc(L, **dkw), **ckw) == getattr(L, "KAN_ERR_" + code), (dkw, ckw)


def test_empty_batch_forward_returns_ok_without_launch(L):
    """N = 0 on every variant, dtype and degree: the plans (workspace sizes
    of both passes) are well defined and the forwards return without a
    launch."""
    for v in (L.KAN_VARIANT_AUTO, L.KAN_VARIANT_MFMA, L.KAN_VARIANT_GATHER):
        for dt in (L.KAN_F32, L.KAN_BF16):
            for deg in (1, 3, 5):
                for G in (1, 8, 125):
                    if v == L.KAN_VARIANT_MFMA and deg != 3 and G + deg + 1 < 4:
                        continue                             # too few columns for the matrix cores
                    d = desc(L, N=0, variant=v, dtype=dt, degree=deg, G=G)
                    for ps in (0, 1):
                        assert L.lib().kan_workspace_size(ctypes.byref(d), ps) != ctypes.c_size_t(-1).value
                    assert fwd(L, d) == L.KAN_OK
                    assert L.lib().kan_forward_static(ctypes.byref(d), X, C, W, Y, None) == L.KAN_OK


def k_split(tiles_m, tiles_n, nkt, rows_out, row_bytes, esize):
    """The planner's k-split rule, restated: slices of the k range for a
    contraction of tiles_m x tiles_n output tiles over `nkt` k-tiles whose
    fp32 output has rows_out rows of row_bytes.  Estimate: rounds of 256
    one-per-CU workgroups x k-tiles per workgroup at 2 us (bf16) or 8 us
    (fp32), plus 2P + 1 passes over the partials at 4 bytes/ns.  Either every
    tile row is cut into P slices, or the tile rows that fill whole rounds run
    whole and only the last `tail` rows are cut, into P slices that fit the
    final round.  Taken when it saves >= 1/16, >= 8 k-tiles a slice.
    Returns (slices, k-tiles per slice, tail tile rows)."""
    kt_ns = 2000 if esize == 2 else 8000
    tiles = tiles_m * tiles_n

    def est(P):
        per, rounds = (nkt + P - 1) // P, (tiles * P + 255) // 256
        return rounds * per * kt_ns + ((2 * P + 1) * rows_out * row_bytes // 4000 if P > 1 else 0)
    e1 = est(1)
    best, tb = (1, 0), e1
    P = 2
    while P <= 8 and (nkt + P - 1) // P >= 8:
        if est(P) < tb:
            best, tb = (P, tiles_m), est(P)
        P += 1
    full = tiles // 256
    if full >= 1:
        h = full * 256 // tiles_n
        t = tiles_m - h
        P = min(8, 256 // (t * tiles_n), nkt // 8) if t > 0 else 0
        if P >= 2:
            per = (nkt + P - 1) // P
            e = ((h * tiles_n + 255) // 256 * nkt * kt_ns + per * kt_ns
                 + (2 * P + 1) * max(0, rows_out - 256 * h) * row_bytes // 4000)
            if e < tb:
                best, tb = (P, t), e
    if tb > e1 - e1 // 16:
        best = (1, 0)
    if best[0] == 1:
        return 1, nkt, 0
    nks = (nkt + best[0] - 1) // best[0]
    return (nkt + nks - 1) // nks, nks, best[1]


def test_k_split_choices():
    """The split the rule gives the workloads' launches: the 768 -> 3072
    layer on 12608 rows (bf16, G = 5, base) runs its forward (50 x 12
    tiles, 108 k-tiles) as 42 whole tile rows and the last 8 in 2 slices,
    its dC (12 x 27 tiles, 200 k-tiles) as 9 whole rows and 3 in 3 slices;
    the 3072 -> 768 layer's dC (3 x 108) as 2 whole rows and 1 in 2
    slices, its forward (50 x 3 tiles, 432 k-tiles) every tile in 5
    slices; the 4096 -> 4096 layer on 65536 rows fills whole rounds and
    stays whole; the tail test's dC shapes (17 x 17 tiles) slice their last
    2 tile rows."""
    assert k_split(50, 12, 108, 12608, 3072 * 4, 2) == (2, 54, 8)
    assert k_split(12, 27, 200, 3072, 768 * 9 * 4, 2) == (3, 67, 3)
    assert k_split(3, 108, 200, 768, 3072 * 9 * 4, 2) == (2, 100, 1)
    assert k_split(50, 3, 432, 12608, 768 * 4, 2) == (5, 87, 50)
    assert k_split(256, 16, 1536, 65536, 4096 * 4, 2) == (1, 1536, 0)
    assert k_split(16, 384, 1024, 4096, 4096 * 24 * 4, 2) == (1, 1024, 0)
    assert k_split(17, 17, 16, 4302, 342 * 12 * 4, 2)[2] == 2
    assert k_split(17, 17, 32, 4302, 342 * 12 * 4, 4)[2] == 2


def split_bytes(tiles_m, tiles_n, nkt, rows_out, row_bytes, esize, f32_forward=False):
    """Bytes of the partial outputs of a k-split contraction (0 when not
    split): P slices of the tail rows' output.  A float32 forward sums in
    slices of at most 8 k-tiles on every tile row."""
    P, nks, tail = k_split(tiles_m, tiles_n, nkt, rows_out, row_bytes, esize)
    if f32_forward and nkt > 8 and not (P > 1 and tail == tiles_m and nks <= 8):
        P, tail = (nkt + 7) // 8, tiles_m
    if P <= 1:
        return 0
    rows = rows_out - (tiles_m - tail) * 256
    return (P * rows * row_bytes + 255) // 256 * 256


def gather_fwd_ws(N, I, O, K, D, base):
    """Workspace of the local-gather forward: float64 partial outputs of its
    input slices, used when its blocks (R rows x 64 outputs) are fewer than
    the 256 CUs and the layer has at least 2^16 edge-rows."""
    ob = (O + 63) // 64
    nt = 1024 if ((N + 255) // 256 * ob >= 64 or K > 32) else 256
    R = nt // 4
    T = (N + R - 1) // R * ob
    S = 1
    if N * I * O >= 1 << 16 and T < 256:
        S = max(1, min((256 + T - 1) // T, (I + 7) // 8))
    IS = (I + S - 1) // S
    S = (I + IS - 1) // IS
    return (S * N * O * 8 + 255) // 256 * 256 if S > 1 else 0


def gather_bwd_ws(N, I, O, K, base):
    """Workspace of the local-gather backward: float32 partial dx of its
    output slices (256-row x 16-input blocks) and partial dC / dW_base of its
    row slices (one input per wave, 64 outputs), each used when its blocks
    are fewer than the 256 CUs and the layer has at least 2^16 edge-rows."""
    big = N * I * O >= 1 << 16
    r = lambda a, b: (a + b - 1) // b * b
    jc = 4
    for c in (16, 8):
        if 2 * (256 * c + 16 * K * (c + 4) + 16 * (c + 4)) * 4 <= 150 * 1024:
            jc = c
            break
    T = (N + 255) // 256 * ((I + 15) // 16)
    sx = max(1, min((256 + T - 1) // T, (O + 4 * jc - 1) // (4 * jc))) if big and T < 256 else 1
    js = r((O + sx - 1) // sx, jc)
    sx = (O + js - 1) // js
    kmax = 16 if K <= 16 else 32 if K <= 32 else 64 if K <= 64 else 132
    opl = 2 if kmax <= 32 and O > 64 else 1
    nw = (1024 if kmax * opl <= 64 else 512) // 64
    T = (I + nw - 1) // nw * ((O + 64 * opl - 1) // (64 * opl))
    sc = max(1, min((256 + T - 1) // T, (N + 127) // 128)) if big and T < 256 else 1
    rs = max(64, r((N + sc - 1) // sc, 64))
    sc = max(1, (N + rs - 1) // rs)
    ws = r(sx * N * I * 4, 256) if sx > 1 else 0
    if sc > 1:
        ws += r(sc * O * I * K * 4, 256) + (r(sc * O * I * 4, 256) if base else 0)
    return ws


def auto_bwd_gather(N, I, O, Kb):
    """float32 AUTO backward: gather when its estimate (N I O / 1.6e12 s) is
    below the dense contractions' (4 N I O Kb / 110e12 s + 150 us)."""
    nio = float(N) * I * O
    return not (4.0 * nio * Kb / 110e12 + 150e-6 < nio / 1.6e12)


def test_workspace_sizes(L):
    ws = lambda **kw: L.lib().kan_workspace_size(ctypes.byref(desc(L, **kw)), 0)
    wb = lambda **kw: L.lib().kan_workspace_size(ctypes.byref(desc(L, **kw)), 1)
    assert ws(variant=L.KAN_VARIANT_GATHER) == 0 and wb(variant=L.KAN_VARIANT_GATHER) == 0
    for (N, I, O, G, base) in [(1024, 784, 64, 8, 1), (1024, 64, 10, 8, 1), (8192, 1024, 1024, 50, 0),
                               (300, 5000, 7, 20, 1), (5000, 3, 300, 125, 1), (64, 16, 8, 8, 1)]:
        assert wb(N=N, I=I, O=O, G=G, has_base=base, variant=L.KAN_VARIANT_GATHER) == \
            gather_bwd_ws(N, I, O, G + 3, base)
    assert gather_bwd_ws(1024, 784, 64, 11, 1) > 0                # the quick-start layer splits
    # MFMA forward: packed C' [O padded to 256][I*Kb padded to the k-tile]
    r = lambda a, b: (a + b - 1) // b * b
    for dt, es, bk in [(L.KAN_F32, 4, 32), (L.KAN_BF16, 2, 64)]:
        for (N, I, O, G, base) in [(64, 16, 8, 8, 1), (1000, 777, 300, 20, 0), (5, 3, 2, 1, 1),
                                   (12608, 768, 3072, 5, 1), (12608, 3072, 768, 5, 1), (8192, 1024, 1024, 50, 0),
                                   (300, 40, 2000, 8, 1), (700, 100, 1793, 3, 0), (65536, 4096, 4096, 5, 1)]:
            Kb = G + 3 + base
            # bf16 forwards with 11 <= Kb <= 32 whose 2:4 layout (NG groups of 4
            # columns per input) costs <= 3/4 of the dense one pack I * 4 NG columns
            ng = max(4, (Kb + 3) // 4)
            ng += ng & 1
            sparse = dt == L.KAN_BF16 and ng <= 8 and Kb >= 11 and 8 * ng <= 3 * Kb
            Op, Np = r(O, 256), r(N, 256)
            # bf16 layers with Kb <= 12 build the dense basis operand once:
            # the forward's ([Np][I Kb padded to 64]) from 8 output tiles,
            # dC's ([I Kb padded to 256][Np]) from 3
            fits = dt == L.KAN_BF16 and Kb <= 12 and Np * r(I * Kb, 256) * 2 <= 1 << 30
            mat, mat_dc = fits and Op // 256 >= 8, fits and Op // 256 >= 3

            def fwd_bytes(kf, nkt, basis=False):
                # packed C', the built basis, then the partial y of a split forward
                return (r(Op * kf * es, 256) + (r(Np * kf * es, 256) if basis else 0)
                        + split_bytes(Np // 256, Op // 256, nkt, N, O * 4, es, es == 4))
            kf = r(I * 4 * ng, 64) if sparse else r(I * Kb, bk)
            assert ws(N=N, I=I, O=O, G=G, has_base=base, dtype=dt) == \
                fwd_bytes(kf, kf // (64 if sparse else bk), mat and not sparse)
            if dt == L.KAN_BF16:
                # the truncated-power forward packs the dense operand
                assert L.lib().kan_workspace_size(ctypes.byref(desc(
                    L, N=N, I=I, O=O, G=G, has_base=base, dtype=dt, flags=L.KAN_FLAG_TP_FORWARD)), 0) == \
                    fwd_bytes(r(I * Kb, bk), r(I * Kb, bk) // bk)
            if sparse:
                assert L.lib().kan_workspace_size(ctypes.byref(desc(
                    L, N=N, I=I, O=O, G=G, has_base=base, dtype=dt, flags=L.KAN_FLAG_DENSE_FORWARD)), 0) == \
                    fwd_bytes(r(I * Kb, bk), r(I * Kb, bk) // bk, mat)
            tiles = (I * Kb + 255) // 256           # dx tiles of 256 P columns
            want = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 2 * 4, 256)
            want += r(tiles * 256 * Np * es, 256) if mat_dc else 0
            want += split_bytes(Op // 256, tiles, Np // bk, O, I * Kb * 4, es)   # dC over batch slices
            assert wb(N=N, I=I, O=O, G=G, has_base=base, dtype=dt) == want
    # auto: bf16 on the matrix cores; float32 forward on the gather kernel and
    # backward on the matrix cores
    assert ws(G=125, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) > 0      # largest grid: MFMA fits
    assert ws(G=126, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) == ctypes.c_size_t(-1).value
    # float32 AUTO: gather forward (no workspace unless it splits its
    # inputs), matrix-core backward
    assert ws(variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_F32) == 0
    for (N, I, O, G, base) in [(1024, 784, 64, 8, 1), (1024, 64, 10, 8, 1), (32, 8, 4, 8, 0), (8192, 1024, 1024, 50, 0),
                               (300, 5000, 7, 20, 1), (1, 100000, 1, 3, 0)]:
        for v in (L.KAN_VARIANT_AUTO, L.KAN_VARIANT_GATHER):
            assert ws(N=N, I=I, O=O, G=G, has_base=base, variant=v, dtype=L.KAN_F32) == \
                gather_fwd_ws(N, I, O, G + 3, 3, base)
    assert gather_fwd_ws(1024, 784, 64, 11, 3, 1) > 0            # the 784-wide quick-start layer splits
    # float32 AUTO backward by the cost estimate: gather for the quick-start
    # layers and the G = 20 / 50 grid sweep, matrix cores for the 1024-wide
    # layer at G = 8
    for (N, I, O, G, base) in [(1024, 784, 64, 8, 1), (1024, 64, 10, 8, 1), (32, 8, 4, 8, 0),
                               (8192, 1024, 1024, 8, 0), (8192, 1024, 1024, 20, 0), (8192, 1024, 1024, 50, 0)]:
        g = auto_bwd_gather(N, I, O, G + 3 + base)
        want = wb(N=N, I=I, O=O, G=G, has_base=base, dtype=L.KAN_F32,
                  variant=L.KAN_VARIANT_GATHER if g else L.KAN_VARIANT_MFMA)
        assert wb(N=N, I=I, O=O, G=G, has_base=base, variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_F32) == want
    assert auto_bwd_gather(1024, 784, 64, 12) and auto_bwd_gather(8192, 1024, 1024, 23)
    assert not auto_bwd_gather(8192, 1024, 1024, 11)
    assert ws(variant=L.KAN_VARIANT_AUTO, dtype=L.KAN_BF16) == ws(variant=L.KAN_VARIANT_MFMA,
                                                                   dtype=L.KAN_BF16) > 0


def test_built_basis_thresholds(L):
    """The built basis operands start exactly where the planner's rule puts
    them: dC's from 3 output tiles (O = 513), the forward's from 8
    (O = 1793, dense forward), bf16 only, Kb <= 12 only, and not past
    1 GiB."""
    r = lambda a, b: (a + b - 1) // b * b

    def want(N, I, O, G, dt, built):
        es, bk = (2, 64) if dt == L.KAN_BF16 else (4, 32)
        Kb = G + 4
        Op, Np = r(O, 256), r(N, 256)
        tiles = (I * Kb + 255) // 256
        kf = r(I * Kb, bk)
        f = (r(Op * kf * es, 256) + (r(Np * kf * es, 256) if built[0] else 0)
             + split_bytes(Np // 256, Op // 256, kf // bk, N, O * 4, es, es == 4))
        b = (r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 2 * 4, 256)
             + (r(tiles * 256 * Np * es, 256) if built[1] else 0)
             + split_bytes(Op // 256, tiles, Np // bk, O, I * Kb * 4, es))
        return f, b

    def got(N, I, O, G, dt):
        d = desc(L, N=N, I=I, O=O, G=G, has_base=1, dtype=dt, flags=L.KAN_FLAG_DENSE_FORWARD)
        return L.lib().kan_workspace_size(ctypes.byref(d), 0), L.lib().kan_workspace_size(ctypes.byref(d), 1)

    bf, f32 = L.KAN_BF16, L.KAN_F32
    for O, built in [(512, (False, False)), (513, (False, True)), (1792, (False, True)), (1793, (True, True))]:
        assert got(1000, 40, O, 8, bf) == want(1000, 40, O, 8, bf, built), O          # Kb = 12
    assert got(1000, 40, 1793, 9, bf) == want(1000, 40, 1793, 9, bf, (False, False))  # Kb = 13
    assert got(1000, 40, 1793, 8, f32) == want(1000, 40, 1793, 8, f32, (False, False))
    # 65536 x 4096 inputs at Kb = 9 is 4.8 GB of basis: past 1 GiB
    assert got(65536, 4096, 4096, 5, bf) == want(65536, 4096, 4096, 5, bf, (False, False))


def test_workspace_sizes_other_degrees(L):
    """Degree D != 3: K = G + D columns per input and the cubic layer's
    choice of kernels (AUTO: bf16 on the matrix cores; float32 forward on the
    gather kernel, backward on the matrix cores from 2^16 edge-rows), never
    the structured-sparse forward, otherwise the cubic layout."""
    r = lambda a, b: (a + b - 1) // b * b
    for dt, es, bk in [(L.KAN_F32, 4, 32), (L.KAN_BF16, 2, 64)]:
        for (N, I, O, G, base, D) in [(64, 16, 8, 8, 1, 1), (1000, 77, 300, 20, 0, 5), (12608, 768, 3072, 5, 1, 2),
                                      (5, 3, 2, 1, 1, 4), (1024, 784, 64, 8, 1, 2)]:
            Kb = G + D + base
            Op, Np = r(O, 256), r(N, 256)
            kf = r(I * Kb, bk)
            want_f = r(Op * kf * es, 256) + split_bytes(Np // 256, Op // 256, kf // bk, N, O * 4, es, es == 4)
            tiles = (I * Kb + 255) // 256
            want_b = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 2 * 4, 256)
            want_b += split_bytes(Op // 256, tiles, Np // bk, O, I * Kb * 4, es)
            for v in (L.KAN_VARIANT_AUTO, L.KAN_VARIANT_MFMA, L.KAN_VARIANT_GATHER):
                d = desc(L, N=N, I=I, O=O, G=G, has_base=base, dtype=dt, degree=D, variant=v)
                gather_f = v == L.KAN_VARIANT_GATHER or (v == L.KAN_VARIANT_AUTO and dt == L.KAN_F32)
                gather_b = v == L.KAN_VARIANT_GATHER or (v == L.KAN_VARIANT_AUTO and dt == L.KAN_F32
                                                         and auto_bwd_gather(N, I, O, Kb))
                assert L.lib().kan_workspace_size(ctypes.byref(d), 0) == (
                    gather_fwd_ws(N, I, O, G + D, D, base) if gather_f else want_f)
                assert L.lib().kan_workspace_size(ctypes.byref(d), 1) == (
                    gather_bwd_ws(N, I, O, G + D, base) if gather_b else want_b)
    # too few columns for the matrix cores (degree 1, G = 1, no base branch:
    # 2 per input): AUTO takes the gather kernels in both dtypes
    for dt in (L.KAN_F32, L.KAN_BF16):
        d = desc(L, N=64, I=16, O=8, G=1, has_base=0, dtype=dt, degree=1, variant=L.KAN_VARIANT_AUTO)
        assert L.lib().kan_workspace_size(ctypes.byref(d), 0) == 0
        assert L.lib().kan_workspace_size(ctypes.byref(d), 1) == 0


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


GROUP_BAD_DESCS = [
    (dict(N=-1), -2), (dict(I=0), -2), (dict(groups=0), -2), (dict(groups=301), -2),
    (dict(N=1 << 40), -2), (dict(G=0), -3), (dict(G=126), -3), (dict(lo=1.0, hi=1.0), -3),
    (dict(lo=float("nan")), -3), (dict(dtype=2), -4), (dict(degree=2), -8)]


@pytest.mark.parametrize("kw,code", GROUP_BAD_DESCS)
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
        for (N, P, O, G) in [(100, 8, 20, 5), (8192, 512, 1024, 5), (300, 7, 33, 8), (5, 3, 2, 1), (64, 16, 700, 1),
                             (77, 4, 300, 13)]:
            Kb = (G + 3) ** 2
            Op, Np = r(O, 256), r(N, 256)
            kf = r(P * Kb, bk)
            want_f = r(Op * kf * es, 256) + split_bytes(Np // 256, Op // 256, kf // bk, N, O * 4, es, es == 4)
            tiles = (P * Kb + 255) // 256
            want_b = r(tiles * 256 * Op * es, 256) + 2 * r(Np * Op * es, 256) + r(Np * tiles * 4 * 4, 256)
            # bf16 dC from 3 output tiles: the pair basis built once, [tiles * 256][Np]
            if dt == 1 and Op // 256 >= 3 and Np * r(P * Kb, 256) * 2 <= 1 << 30:
                want_b += r(tiles * 256 * Np * es, 256)
            want_b += split_bytes(Op // 256, tiles, Np // bk, O, P * Kb * 4, es)
            d = sdesc(L, N=N, P=P, O=O, G=G, dtype=dt)
            assert L.lib().kan_surface_workspace_size(ctypes.byref(d), 0) == want_f
            assert L.lib().kan_surface_workspace_size(ctypes.byref(d), 1) == want_b
    bad = ctypes.c_size_t(-1).value
    assert L.lib().kan_surface_workspace_size(ctypes.byref(sdesc(L)), 2) == bad
    assert L.lib().kan_surface_workspace_size(None, 0) == bad


SURFACE_BAD_DESCS = [
    (dict(N=-1), -2), (dict(P=0), -2), (dict(O=0), -2), (dict(G=0), -3), (dict(G=14), -3),
    (dict(lo=1.0, hi=0.5), -3), (dict(hi=float("inf")), -3), (dict(dtype=5), -4), (dict(degree=1), -8),
    (dict(flags=4), -8), (dict(P=1 << 30), -2)]


@pytest.mark.parametrize("kw,code", SURFACE_BAD_DESCS)
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
