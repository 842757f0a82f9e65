// C ABI of the KAN layer library: argument validation, the per-call plan and
// workspace layout, and kernel dispatch.  Every check runs before the first
// launch, so a call that fails has enqueued nothing.  No C++ exception leaves
// this file; there is no mutable global state.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "kan_internal.h"

namespace kan {

namespace {

constexpr int64_t kIndexLimit = (int64_t(1) << 31) - 4096;  // keeps 32-bit tile math safe
constexpr int kMaxG = 125;                                      // K = G + 3 <= 128
constexpr int64_t kF32SliceTiles = 8;                           // float32 forward: k-tiles per slice

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    const void* p;
    size_t n;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

int status_of(hipError_t e) { return e == hipSuccess ? KAN_OK : KAN_ERR_HIP; }

// Whether a dense bf16 cubic layer builds a basis operand once in HBM
// rather than in every workgroup that needs it.  Inside the contraction
// every output tile regenerates the basis tiles of its k range; with few
// columns per input (Kb <= 12: 21 or more inputs per 256-column tile) that
// generator work exceeds what loading a built tile costs (the 768 -> 3072
// -> 768 channel mixer on 12608 rows, Kb = 9: about 2.2 (forward) and 2.5
// (dC) against 1.6-1.8 us per k-tile of a workgroup).  Building costs one
// write of the N x I Kb bf16 basis, repaid when enough output tiles read
// each of its tiles: measured on that mixer, the forward gains with 12
// reading tiles and loses with 3; dC gains with 12 and with 3.  So the forward's operand is built from 8 output tiles
// (O > 1792) and dC's from 3 (O > 512); the array is kept within 1 GiB.
// The 2-D layer's dC generator (16 products per pair) costs more than a
// load at any pair width, so its dC operand is built by the same rule.
bool materialize_basis(const Plan& q, int64_t min_tiles) {
    const int64_t bytes = q.Npad * round_up(q.IKb, 256) * 2;
    return q.dtype == KAN_BF16 && q.degree == 3 && !q.tp && (q.pair || q.Kb <= 12) &&
           q.Opad / kTileN >= min_tiles && bytes <= (int64_t(1) << 30);
}

// Matrix-core geometry and workspace layout of a plan whose shape, K, Kb,
// base, dtype and per-pass variants are set.
void plan_layout(Plan& q, bool dense_forward, bool materialize) {
    if (q.variant_fwd != KAN_VARIANT_MFMA && q.variant_bwd != KAN_VARIANT_MFMA) return;
    q.BK = kTileKBytes / q.esize;
    q.IKb = q.I * q.Kb;
    q.Opad = round_up(q.O, kTileN);
    q.Npad = round_up(std::max<int64_t>(q.N, 1), kTileM);
    q.Kf = round_up(q.IKb, q.BK);
    q.tiles_dx = (q.IKb + kTileN - 1) / kTileN;
    size_t off = 0;
    auto take = [&](size_t bytes, size_t* o, size_t* sz) {
        *o = off;
        *sz = bytes;
        off += (size_t)round_up((int64_t)bytes, 256);
    };
    // Sparse forward: NG = ceil(Kb / 4) groups, at least 4 (so that 4
    // consecutive columns land in 4 groups) and even (so that an input's
    // index nibbles fill whole bytes); taken when its padded width costs
    // at most 3/4 of the dense contraction.
    int ng = std::max(4, (q.Kb + 3) / 4);
    ng += ng & 1;
    q.sparse = q.dtype == KAN_BF16 && !dense_forward && !q.pair && q.degree == 3 && ng <= 8 && q.Kb >= 11 &&
               8 * ng <= 3 * q.Kb && q.I * 4 * ng <= kIndexLimit;
    q.NG = ng;
    q.Kb8 = 4 * ng;
    if (q.pair) {
        // 2-D layer: the sparse form exists for K1 = 8 (G = 5), a pair's 64
        // columns in one k-tile, permuted but not widened
        q.sparse = q.dtype == KAN_BF16 && !dense_forward && q.Kb == 64;
        q.NG = 0;
        q.Kb8 = 64;
    }
    q.Kfs = round_up(q.I * q.Kb8, 64);
    take((size_t)(q.Opad * (q.sparse ? q.Kfs : q.Kf)) * q.esize, &q.off_cp, &q.sz_cp);
    q.mat_fwd = materialize && !q.sparse && !q.pair && materialize_basis(q, 8);
    if (q.mat_fwd) take((size_t)(q.Npad * q.Kf) * q.esize, &q.off_phi, &q.sz_phi);
    const int64_t nkt_fwd = q.sparse ? q.Kfs / 64 : q.Kf / q.BK;
    const KSplit kf = k_split(q.Npad / kTileM, q.Opad / kTileN, nkt_fwd, q.N, q.O * 4, q.esize);
    q.split_fwd = kf.P;
    q.nks_fwd = kf.nks;
    q.tail_fwd = kf.tail;
    // A float32 forward sums its contraction in slices of at most 8 k-tiles
    // (256 terms): a float32 running sum over the whole basis row (9408
    // terms at 784 inputs) loses accuracy that the next layer's B' amplifies;
    // the slices' partials are added in float64.
    const bool sliced = q.split_fwd > 1 && q.tail_fwd == q.Npad / kTileM && q.nks_fwd <= kF32SliceTiles;
    if (q.dtype == KAN_F32 && nkt_fwd > kF32SliceTiles && !sliced) {
        q.nks_fwd = kF32SliceTiles;
        q.split_fwd = (int)((nkt_fwd + kF32SliceTiles - 1) / kF32SliceTiles);
        q.tail_fwd = q.Npad / kTileM;
    }
    if (q.split_fwd > 1)
        take((size_t)(q.split_fwd * fwd_tail_rows(q) * q.O) * 4, &q.off_yp, &q.sz_yp);
    q.ws_fwd = q.variant_fwd == KAN_VARIANT_MFMA ? off : 0;
    off = 0;
    take((size_t)(q.tiles_dx * kTileN * q.Opad) * q.esize, &q.off_cpt, &q.sz_cpt);
    take((size_t)(q.Npad * q.Opad) * q.esize, &q.off_dyp, &q.sz_dyp);
    take((size_t)(q.Opad * q.Npad) * q.esize, &q.off_dyt, &q.sz_dyt);
    take((size_t)(q.Npad * q.tiles_dx * 2 * (q.pair ? 2 : 1)) * 4, &q.off_part, &q.sz_part);
    q.mat_dc = materialize && materialize_basis(q, 3);
    if (q.mat_dc) take((size_t)(q.tiles_dx * kTileN * q.Npad) * q.esize, &q.off_phit, &q.sz_phit);
    const KSplit kc = k_split(q.Opad / kTileM, (q.IKb + kTileN - 1) / kTileN, q.Npad / q.BK, q.O, q.I * q.Kb * 4,
                              q.esize);
    q.split_dc = kc.P;
    q.nks_dc = kc.nks;
    q.tail_dc = kc.tail;
    if (q.split_dc > 1) take((size_t)(q.split_dc * dc_tail_rows(q) * q.I * q.Kb) * 4, &q.off_dcp, &q.sz_dcp);
    q.ws_bwd = q.variant_bwd == KAN_VARIANT_MFMA ? off : 0;
}

// degree 1 .. 5 when any_degree, else 3 only
int grid_check(const kan_grid_t& g, int max_G, bool any_degree) {
    if (any_degree ? (g.degree < 1 || g.degree > 5) : g.degree != 3) return KAN_ERR_UNSUPPORTED;
    if (g.G < 1 || g.G > max_G) return KAN_ERR_GRID;
    if (!isfinite(g.lo) || !isfinite(g.hi) || !(g.lo < g.hi)) return KAN_ERR_GRID;
    return KAN_OK;
}

// knot units measured from t_0 = lo - degree h
void grid_constants(Plan& q, const kan_grid_t& g) {
    const double lo = g.lo, hi = g.hi;
    q.G = g.G;
    q.degree = g.degree;
    q.gk.scale = (float)((double)q.G / (hi - lo));
    q.gk.shift = (float)((double)g.degree - lo * (double)q.G / (hi - lo));
    q.gk.G = q.G;
}

}  // namespace

int make_plan_surface(const kan_surface_desc_t* d, Plan* p) {
    if (!d || !p) return KAN_ERR_NULL;
    if (d->N < 0 || d->P < 1 || d->O < 1) return KAN_ERR_SHAPE;
    // a pair's (G+3)^2 columns must fit one 256-wide tile
    int st = grid_check(d->grid, 13, false);
    if (st != KAN_OK) return st;
    if (d->dtype != KAN_F32 && d->dtype != KAN_BF16) return KAN_ERR_DTYPE;
    if (d->flags & ~(KAN_FLAG_PREPARED | KAN_FLAG_DENSE_FORWARD)) return KAN_ERR_UNSUPPORTED;
    Plan q;
    memset(&q, 0, sizeof(q));
    q.pair = 1;
    q.N = d->N;
    q.I = d->P;
    q.xI = 2 * d->P;
    q.O = d->O;
    grid_constants(q, d->grid);
    q.K = (q.G + 3) * (q.G + 3);
    q.base = 0;
    q.Kb = q.K;
    q.dtype = d->dtype;
    q.esize = d->dtype == KAN_F32 ? 4 : 2;
    if (q.N > kIndexLimit || q.O > kIndexLimit || q.xI > kIndexLimit || q.I * q.Kb > kIndexLimit)
        return KAN_ERR_SHAPE;
    q.variant_fwd = q.variant_bwd = KAN_VARIANT_MFMA;
    plan_layout(q, (d->flags & KAN_FLAG_DENSE_FORWARD) != 0, true);
    *p = q;
    return KAN_OK;
}

int make_plan(const kan_desc_t* d, Plan* p, bool materialize) {
    if (!d || !p) return KAN_ERR_NULL;
    if (d->N < 0 || d->I < 1 || d->O < 1) return KAN_ERR_SHAPE;
    // G <= kMaxG: the gather kernels stage an input's K = G+3 coefficients
    // for a tile of outputs in LDS, which holds 128 of them
    const int gst = grid_check(d->grid, kMaxG, true);
    if (gst != KAN_OK) return gst;
    if (d->dtype != KAN_F32 && d->dtype != KAN_BF16) return KAN_ERR_DTYPE;
    if (d->has_base != 0 && d->has_base != 1) return KAN_ERR_UNSUPPORTED;
    if (d->variant < KAN_VARIANT_AUTO || d->variant > KAN_VARIANT_GATHER) return KAN_ERR_UNSUPPORTED;
    if (d->flags & ~(KAN_FLAG_PREPARED | KAN_FLAG_DENSE_FORWARD | KAN_FLAG_TP_FORWARD))
        return KAN_ERR_UNSUPPORTED;

    Plan q;
    memset(&q, 0, sizeof(q));
    q.N = d->N;
    q.I = d->I;
    q.xI = d->I;
    q.O = d->O;
    grid_constants(q, d->grid);
    q.K = q.G + q.degree;
    q.base = d->has_base;
    q.Kb = q.K + q.base;
    q.dtype = d->dtype;
    q.esize = d->dtype == KAN_F32 ? 4 : 2;
    if (q.N > kIndexLimit || q.O > kIndexLimit || q.I * q.Kb > kIndexLimit) return KAN_ERR_SHAPE;

    // An input's Kb columns must fit one 256-wide tile on the matrix cores,
    // and a degree other than 3 needs at least 4 columns per input (the
    // operand generators' instances cover that many inputs per tile).
    // AUTO: bf16 runs both passes on the matrix cores.  float32 runs the
    // forward on the local gather kernel, whose sums over inputs are float64
    // and which touches only the D + 1 non-zero basis functions.  Its
    // backward takes whichever of the two kernel families the measured rates
    // make faster: the gather dx and dC together do about 1.6e12 edge-rows
    // (N I O) per second whatever K is; the two dense float32 contractions
    // execute 4 N I O Kb flops at about 110 TFLOP/s, plus about 150 us of
    // packing, epilogues and launches.  So the gather backward wins from Kb of
    // about 17 up, and on small layers at any Kb.
    const bool mfma_ok = q.Kb <= kTileN && (q.degree == 3 || q.Kb >= 4);
    if (d->variant == KAN_VARIANT_MFMA && !mfma_ok) return KAN_ERR_UNSUPPORTED;
    if (d->variant == KAN_VARIANT_GATHER) {
        q.variant_fwd = q.variant_bwd = KAN_VARIANT_GATHER;
    } else if (d->variant == KAN_VARIANT_MFMA) {
        q.variant_fwd = q.variant_bwd = KAN_VARIANT_MFMA;
    } else {
        q.variant_fwd = (mfma_ok && q.dtype == KAN_BF16) ? KAN_VARIANT_MFMA : KAN_VARIANT_GATHER;
        const double nio = (double)q.N * (double)q.I * (double)q.O;
        const double t_gather = nio / 1.6e12, t_mfma = 4.0 * nio * q.Kb / 110e12 + 150e-6;
        q.variant_bwd = mfma_ok && (q.dtype == KAN_BF16 || t_mfma < t_gather) ? KAN_VARIANT_MFMA
                                                                               : KAN_VARIANT_GATHER;
    }

    // the truncated-power generator: the dense bf16 forward of a cubic layer
    // on the matrix cores (in float32 its alternating sum loses ~2e-6 per
    // basis value, more than a chain of layers leaves room for)
    const bool tp = (d->flags & KAN_FLAG_TP_FORWARD) != 0;
    if (tp && (q.dtype != KAN_BF16 || q.degree != 3 || q.variant_fwd != KAN_VARIANT_MFMA))
        return KAN_ERR_UNSUPPORTED;
    q.tp = tp;
    plan_layout(q, tp || (d->flags & KAN_FLAG_DENSE_FORWARD) != 0, materialize);
    if (q.variant_fwd == KAN_VARIANT_GATHER) {
        q.gf = gather_fwd_plan(q.N, q.I, q.O, q.K, q.degree, q.base);
        q.ws_fwd = q.gf.ws;
    }
    if (q.variant_bwd == KAN_VARIANT_GATHER) {
        q.gb = gather_bwd_plan(q.N, q.I, q.O, q.K, q.base);
        q.ws_bwd = q.gb.ws;
    }
    *p = q;
    return KAN_OK;
}

}  // namespace kan

using namespace kan;

extern "C" {

int kan_abi_version(void) { return KAN_ABI_VERSION; }

const char* kan_status_string(int status) {
    switch (status) {
        case KAN_OK: return "ok";
        case KAN_ERR_NULL: return "required pointer is NULL (or a forbidden one is not)";
        case KAN_ERR_SHAPE: return "invalid shape";
        case KAN_ERR_GRID: return "invalid grid (G < 1 or > 125 (2-D layer: 13), lo >= hi, or non-finite)";
        case KAN_ERR_DTYPE: return "unsupported dtype";
        case KAN_ERR_ALIGN: return "pointer not aligned (tensors 16 bytes, workspace 256)";
        case KAN_ERR_WORKSPACE: return "workspace too small";
        case KAN_ERR_HIP: return "HIP launch failed";
        case KAN_ERR_UNSUPPORTED: return "unsupported option (degree, variant, flags, pass)";
        case KAN_ERR_ALIAS: return "an output overlaps an input or another output";
        default: return "unknown status";
    }
}

size_t kan_workspace_size(const kan_desc_t* desc, int pass) {
    Plan p;
    if (make_plan(desc, &p) != KAN_OK) return SIZE_MAX;
    if (pass != KAN_PASS_FORWARD && pass != KAN_PASS_BACKWARD) return SIZE_MAX;
    return pass == KAN_PASS_FORWARD ? p.ws_fwd : p.ws_bwd;
}

static int pass_variant(const Plan& p, int pass) {
    return pass == KAN_PASS_FORWARD ? p.variant_fwd : p.variant_bwd;
}

static int check_ws(const Plan& p, int pass, const void* ws, size_t ws_bytes) {
    const size_t need = pass == KAN_PASS_FORWARD ? p.ws_fwd : p.ws_bwd;
    if (ws_bytes < need) return KAN_ERR_WORKSPACE;
    if (need > 0 && !ws) return KAN_ERR_NULL;
    if (ws && !aligned(ws, 256)) return KAN_ERR_ALIGN;
    return KAN_OK;
}

static char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

static int prepare_impl(const Plan& p, int pass, const void* C, const void* W, const float* dy,
                        void* ws, hipStream_t s) {
    if (pass_variant(p, pass) != KAN_VARIANT_MFMA) return KAN_OK;
    hipError_t e = hipSuccess;
    if (pass == KAN_PASS_FORWARD) {
        e = p.sparse ? launch_pack_fwd_sparse(p, C, W, ws_at(ws, p.off_cp), s)
                     : launch_pack_fwd(p, C, W, ws_at(ws, p.off_cp), s);
    } else {
        e = launch_pack_bwd(p, C, W, ws_at(ws, p.off_cpt), s);
        if (e == hipSuccess && p.N > 0)
            e = launch_prep_dy(p, dy, ws_at(ws, p.off_dyp), ws_at(ws, p.off_dyt), s);
    }
    return status_of(e);
}

int kan_prepare(const kan_desc_t* desc, int pass, const void* C, const void* W_base,
                const float* dy, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int st = make_plan(desc, &p);
    if (st != KAN_OK) return st;
    if (pass != KAN_PASS_FORWARD && pass != KAN_PASS_BACKWARD) return KAN_ERR_UNSUPPORTED;
    if (!C) return KAN_ERR_NULL;
    if ((W_base != nullptr) != (p.base == 1)) return KAN_ERR_NULL;
    if (pass == KAN_PASS_BACKWARD && p.N > 0 && !dy) return KAN_ERR_NULL;
    if (!aligned(C, 16) || (W_base && !aligned(W_base, 16)) || (dy && !aligned(dy, 16)))
        return KAN_ERR_ALIGN;
    if ((st = check_ws(p, pass, ws, ws_bytes)) != KAN_OK) return st;
    const size_t wsn = pass == KAN_PASS_FORWARD ? p.ws_fwd : p.ws_bwd;
    const Range wr{ws, wsn};
    const Range in[] = {{C, (size_t)(p.O * p.I * p.K) * p.esize},
                        {W_base, (size_t)(p.O * p.I) * p.esize},
                        {dy, pass == KAN_PASS_BACKWARD ? (size_t)(p.N * p.O) * 4 : 0}};
    for (const Range& r : in)
        if (overlap(wr, r)) return KAN_ERR_ALIAS;
    (void)hipGetLastError();
    return prepare_impl(p, pass, C, W_base, dy, ws, (hipStream_t)stream);
}

int kan_forward(const kan_desc_t* desc, const void* x, const void* C, const void* W_base,
                float* y, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int st = make_plan(desc, &p);
    if (st != KAN_OK) return st;
    if ((st = forward_validate(p, x, C, W_base, y, ws, ws_bytes, false)) != KAN_OK) return st;
    return forward_launch(p, desc->flags, x, C, W_base, y, ws, stream);
}

}  // extern "C"

namespace kan {

int forward_validate(const Plan& p, const void* x, const void* C, const void* W_base, const float* y,
                     const void* ws, size_t ws_bytes, bool own_ws) {
    int st;
    if (!C || (p.N > 0 && (!x || !y))) return KAN_ERR_NULL;
    if ((W_base != nullptr) != (p.base == 1)) return KAN_ERR_NULL;
    const void* fptrs[] = {x, C, W_base, y};
    for (const void* q : fptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    if (!own_ws && (st = check_ws(p, KAN_PASS_FORWARD, ws, ws_bytes)) != KAN_OK) return st;
    const Range out{y, (size_t)(p.N * p.O) * 4};
    const Range wr{own_ws ? nullptr : ws, p.ws_fwd};
    const Range in[] = {{x, (size_t)(p.N * p.I) * p.esize},
                        {C, (size_t)(p.O * p.I * p.K) * p.esize},
                        {W_base, (size_t)(p.O * p.I) * p.esize}};
    for (const Range& r : in)
        if (overlap(out, r) || overlap(wr, r)) return KAN_ERR_ALIAS;
    if (overlap(out, wr)) return KAN_ERR_ALIAS;
    return KAN_OK;
}

int forward_launch(const Plan& p, int flags, const void* x, const void* C, const void* W_base, float* y,
                   void* ws, void* stream) {
    if (p.N == 0) return KAN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (p.variant_fwd == KAN_VARIANT_GATHER) return status_of(launch_gather_fwd(p, x, C, W_base, y, ws, s));
    if (!(flags & KAN_FLAG_PREPARED)) {
        const int st = prepare_impl(p, KAN_PASS_FORWARD, C, W_base, nullptr, ws, s);
        if (st != KAN_OK) return st;
    }
    return status_of(launch_mfma_fwd(p, x, ws_at(ws, p.off_cp), ws_at(ws, p.off_phi),
                                     reinterpret_cast<float*>(ws_at(ws, p.off_yp)), y, s));
}

}  // namespace kan

extern "C" {

int kan_backward(const kan_desc_t* desc, const void* x, const void* C, const void* W_base,
                 const float* dy, float* dx, float* dC, float* dW, void* ws, size_t ws_bytes,
                 void* stream) {
    Plan p;
    int st = make_plan(desc, &p);
    if (st != KAN_OK) return st;
    if (!C || (p.N > 0 && (!x || !dy))) return KAN_ERR_NULL;
    if ((W_base != nullptr) != (p.base == 1)) return KAN_ERR_NULL;
    if (dW && !p.base) return KAN_ERR_NULL;
    const void* ptrs[] = {x, C, W_base, dy, dx, dC, dW};
    for (const void* q : ptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    if ((st = check_ws(p, KAN_PASS_BACKWARD, ws, ws_bytes)) != KAN_OK) return st;
    const Range outs[] = {{dx, (size_t)(p.N * p.I) * 4},
                          {dC, (size_t)(p.O * p.I * p.K) * 4},
                          {dW, (size_t)(p.O * p.I) * 4},
                          {ws, p.ws_bwd}};
    const Range ins[] = {{x, (size_t)(p.N * p.I) * p.esize},
                         {C, (size_t)(p.O * p.I * p.K) * p.esize},
                         {W_base, (size_t)(p.O * p.I) * p.esize},
                         {dy, (size_t)(p.N * p.O) * 4}};
    for (int a = 0; a < 4; ++a) {
        for (const Range& r : ins)
            if (overlap(outs[a], r)) return KAN_ERR_ALIAS;
        for (int b = a + 1; b < 4; ++b)
            if (overlap(outs[a], outs[b])) return KAN_ERR_ALIAS;
    }

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (p.N == 0) {  // empty batch: the gradient sums are zero, dx is empty
        hipError_t e = hipSuccess;
        if (dC) e = launch_fill_zero(dC, p.O * p.I * p.K, s);
        if (e == hipSuccess && dW) e = launch_fill_zero(dW, p.O * p.I, s);
        return status_of(e);
    }
    if (p.variant_bwd == KAN_VARIANT_GATHER) {
        hipError_t e = hipSuccess;
        if (dx) e = launch_gather_dx(p, x, C, W_base, dy, dx, ws, s);
        if (e == hipSuccess && (dC || dW)) e = launch_gather_dc(p, x, dy, dC, dW, ws, s);
        return status_of(e);
    }
    if (!(desc->flags & KAN_FLAG_PREPARED)) {
        st = prepare_impl(p, KAN_PASS_BACKWARD, C, W_base, dy, ws, s);
        if (st != KAN_OK) return st;
    }
    hipError_t e = hipSuccess;
    if (dx)
        e = launch_mfma_dx(p, x, ws_at(ws, p.off_dyp), ws_at(ws, p.off_cpt),
                           reinterpret_cast<float*>(ws_at(ws, p.off_part)), dx, s);
    if (e == hipSuccess && (dC || dW))
        e = launch_mfma_dc(p, x, ws_at(ws, p.off_dyt), ws_at(ws, p.off_phit),
                           reinterpret_cast<float*>(ws_at(ws, p.off_dcp)), dC, dW, s);
    return status_of(e);
}

static int basis_eval_impl(const kan_grid_t* grid, int64_t n, int dtype, const void* x, float* B,
                           float* dB, bool truncated_power, void* stream) {
    if (!grid) return KAN_ERR_NULL;
    const int degree = grid->degree;
    int st = grid_check(*grid, kMaxG, true);
    if (st != KAN_OK) return st;
    if (n < 0) return KAN_ERR_SHAPE;
    if (dtype != KAN_F32 && dtype != KAN_BF16) return KAN_ERR_DTYPE;
    const int K = grid->G + degree;
    if (n > kIndexLimit / K) return KAN_ERR_SHAPE;
    if (n == 0) return KAN_OK;
    if (!x || (!B && !dB)) return KAN_ERR_NULL;
    if (!aligned(x, 16) || (B && !aligned(B, 16)) || (dB && !aligned(dB, 16))) return KAN_ERR_ALIGN;
    const size_t ob = (size_t)n * K * 4;
    const Range rx{x, (size_t)n * (dtype == KAN_F32 ? 4 : 2)}, rb{B, ob}, rd{dB, ob};
    if (overlap(rx, rb) || overlap(rx, rd) || overlap(rb, rd)) return KAN_ERR_ALIAS;
    // knot units from t_0 = lo - degree h
    GridK gk;
    const double lo = grid->lo, hi = grid->hi;
    gk.G = grid->G;
    gk.scale = (float)((double)gk.G / (hi - lo));
    gk.shift = (float)((double)degree - lo * (double)gk.G / (hi - lo));
    (void)hipGetLastError();
    return status_of(launch_basis_eval(gk, n, dtype, x, B, dB, truncated_power, degree, (hipStream_t)stream));
}

int kan_basis_eval(const kan_grid_t* grid, int64_t n, int dtype, const void* x, float* B,
                   float* dB, void* stream) {
    return basis_eval_impl(grid, n, dtype, x, B, dB, false, stream);
}

int kan_basis_eval_tp(const kan_grid_t* grid, int64_t n, int dtype, const void* x, float* B,
                      float* dB, void* stream) {
    return basis_eval_impl(grid, n, dtype, x, B, dB, true, stream);
}

size_t kan_surface_workspace_size(const kan_surface_desc_t* desc, int pass) {
    Plan p;
    if (make_plan_surface(desc, &p) != KAN_OK) return SIZE_MAX;
    if (pass != KAN_PASS_FORWARD && pass != KAN_PASS_BACKWARD) return SIZE_MAX;
    return pass == KAN_PASS_FORWARD ? p.ws_fwd : p.ws_bwd;
}

int kan_surface_forward(const kan_surface_desc_t* desc, const void* x, const void* C, float* y, void* ws,
                        size_t ws_bytes, void* stream) {
    Plan p;
    int st = make_plan_surface(desc, &p);
    if (st != KAN_OK) return st;
    if (!C || (p.N > 0 && (!x || !y))) return KAN_ERR_NULL;
    const void* ptrs[] = {x, C, y};
    for (const void* q : ptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    if ((st = check_ws(p, KAN_PASS_FORWARD, ws, ws_bytes)) != KAN_OK) return st;
    const Range out{y, (size_t)(p.N * p.O) * 4};
    const Range wr{ws, p.ws_fwd};
    const Range in[] = {{x, (size_t)(p.N * p.xI) * p.esize}, {C, (size_t)(p.O * p.I * p.K) * p.esize}};
    for (const Range& r : in)
        if (overlap(out, r) || overlap(wr, r)) return KAN_ERR_ALIAS;
    if (overlap(out, wr)) return KAN_ERR_ALIAS;
    if (p.N == 0) return KAN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (!(desc->flags & KAN_FLAG_PREPARED)) {
        st = prepare_impl(p, KAN_PASS_FORWARD, C, nullptr, nullptr, ws, s);
        if (st != KAN_OK) return st;
    }
    return status_of(launch_mfma_fwd(p, x, ws_at(ws, p.off_cp), ws_at(ws, p.off_phi),
                                     reinterpret_cast<float*>(ws_at(ws, p.off_yp)), y, s));
}

int kan_surface_backward(const kan_surface_desc_t* desc, const void* x, const void* C, const float* dy,
                         float* dx, float* dC, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int st = make_plan_surface(desc, &p);
    if (st != KAN_OK) return st;
    if (!C || (p.N > 0 && (!x || !dy))) return KAN_ERR_NULL;
    const void* ptrs[] = {x, C, dy, dx, dC};
    for (const void* q : ptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    if ((st = check_ws(p, KAN_PASS_BACKWARD, ws, ws_bytes)) != KAN_OK) return st;
    const Range outs[] = {{dx, (size_t)(p.N * p.xI) * 4}, {dC, (size_t)(p.O * p.I * p.K) * 4}, {ws, p.ws_bwd}};
    const Range ins[] = {{x, (size_t)(p.N * p.xI) * p.esize},
                         {C, (size_t)(p.O * p.I * p.K) * p.esize},
                         {dy, (size_t)(p.N * p.O) * 4}};
    for (int a = 0; a < 3; ++a) {
        for (const Range& r : ins)
            if (overlap(outs[a], r)) return KAN_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlap(outs[a], outs[b])) return KAN_ERR_ALIAS;
    }
    if (!dx && !dC) return KAN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (p.N == 0) return dC ? status_of(launch_fill_zero(dC, p.O * p.I * p.K, s)) : KAN_OK;
    if (!(desc->flags & KAN_FLAG_PREPARED)) {
        st = prepare_impl(p, KAN_PASS_BACKWARD, C, nullptr, dy, ws, s);
        if (st != KAN_OK) return st;
    }
    hipError_t e = hipSuccess;
    if (dx)
        e = launch_mfma_dx(p, x, ws_at(ws, p.off_dyp), ws_at(ws, p.off_cpt),
                           reinterpret_cast<float*>(ws_at(ws, p.off_part)), dx, s);
    if (e == hipSuccess && dC)
        e = launch_mfma_dc(p, x, ws_at(ws, p.off_dyt), ws_at(ws, p.off_phit),
                           reinterpret_cast<float*>(ws_at(ws, p.off_dcp)),
                           dC, nullptr, s);
    return status_of(e);
}

// Validates a grouped activation; on success *gk and *K describe the grid.
static int group_check(const kan_group_desc_t* d, GridK* gk, int* K, int* esize) {
    if (!d) return KAN_ERR_NULL;
    if (d->grid.degree != 3) return KAN_ERR_UNSUPPORTED;          // the grouped kernels are cubic
    kan_desc_t ld;
    memset(&ld, 0, sizeof(ld));
    ld.N = 1;
    ld.I = 1;
    ld.O = 1;
    ld.grid = d->grid;
    ld.dtype = d->dtype;
    Plan p;
    int st = make_plan(&ld, &p);
    if (st != KAN_OK) return st;
    if (d->N < 0 || d->I < 1 || d->groups < 1 || d->groups > d->I) return KAN_ERR_SHAPE;
    if (d->N > kIndexLimit || d->I * p.K > kIndexLimit) return KAN_ERR_SHAPE;
    *gk = p.gk;
    *K = p.K;
    *esize = p.esize;
    return KAN_OK;
}

size_t kan_group_workspace_size(const kan_group_desc_t* desc) {
    GridK gk;
    int K, es;
    if (group_check(desc, &gk, &K, &es) != KAN_OK) return SIZE_MAX;
    if (desc->N == 0) return 0;
    const GroupPlan gp = grouped_plan(desc->N, desc->I, K);
    return (size_t)round_up((gp.part_floats + gp.red_floats) * 4, 256);
}

int kan_group_forward(const kan_group_desc_t* desc, const void* x, const void* C, float* y,
                      void* stream) {
    GridK gk;
    int K, es;
    int st = group_check(desc, &gk, &K, &es);
    if (st != KAN_OK) return st;
    const int64_t NI = desc->N * desc->I;
    if (!C || (NI > 0 && (!x || !y))) return KAN_ERR_NULL;
    const void* ptrs[] = {x, C, y};
    for (const void* q : ptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    const Range out{y, (size_t)NI * 4};
    if (overlap(out, Range{x, (size_t)NI * es}) || overlap(out, Range{C, (size_t)desc->groups * K * es}))
        return KAN_ERR_ALIAS;
    if (NI == 0) return KAN_OK;
    (void)hipGetLastError();
    return status_of(launch_grouped_fwd(gk, desc->N, desc->I, desc->groups, desc->dtype, x, C, y,
                                        (hipStream_t)stream));
}

int kan_group_backward(const kan_group_desc_t* desc, const void* x, const void* C, const float* dy,
                       float* dx, float* dC, void* ws, size_t ws_bytes, void* stream) {
    GridK gk;
    int K, es;
    int st = group_check(desc, &gk, &K, &es);
    if (st != KAN_OK) return st;
    const int64_t N = desc->N, I = desc->I, NI = N * I;
    if (!C || (N > 0 && (!x || !dy))) return KAN_ERR_NULL;
    const void* ptrs[] = {x, C, dy, dx, dC};
    for (const void* q : ptrs)
        if (q && !aligned(q, 16)) return KAN_ERR_ALIGN;
    const size_t need = dC ? kan_group_workspace_size(desc) : 0;
    if (ws_bytes < need) return KAN_ERR_WORKSPACE;
    if (need > 0 && !ws) return KAN_ERR_NULL;
    if (need > 0 && !aligned(ws, 256)) return KAN_ERR_ALIGN;
    const Range outs[] = {{dx, (size_t)NI * 4}, {dC, (size_t)desc->groups * K * 4}, {ws, need}};
    const Range ins[] = {{x, (size_t)NI * es}, {C, (size_t)desc->groups * K * es}, {dy, (size_t)NI * 4}};
    for (int a = 0; a < 3; ++a) {
        for (const Range& r : ins)
            if (overlap(outs[a], r)) return KAN_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlap(outs[a], outs[b])) return KAN_ERR_ALIAS;
    }
    if (!dx && !dC) return KAN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    float* part = static_cast<float*>(ws);
    float* red = part ? part + grouped_plan(N > 0 ? N : 1, I, K).part_floats : nullptr;
    return status_of(launch_grouped_bwd(gk, N, I, desc->groups, desc->dtype, x, C, dy, dx, dC, part,
                                        red, s));
}

int kan_cast_f32_to_bf16(const float* in, void* out, int64_t n, void* stream) {
    if (n < 0) return KAN_ERR_SHAPE;
    if (n == 0) return KAN_OK;
    if (!in || !out) return KAN_ERR_NULL;
    if (!aligned(in, 16) || !aligned(out, 16)) return KAN_ERR_ALIGN;
    if (overlap(Range{in, (size_t)n * 4}, Range{out, (size_t)n * 2})) return KAN_ERR_ALIAS;
    (void)hipGetLastError();
    return status_of(launch_cast_bf16(in, static_cast<uint16_t*>(out), n, (hipStream_t)stream));
}

}  // extern "C"
