// Host-side launch plans: the k-split of the matrix-core contractions, and
// the block counts, chunk sizes, slices and workspace layouts of the
// local-gather layer kernels and of the grouped activation.  Pure host code (no device code, no HIP calls),
// so the validation and planning path can also be built on its own for the
// host sanitizers.
#include <algorithm>

#include "kan_internal.h"

namespace kan {

// Slices of the k range for a contraction of tiles_m x tiles_n output tiles
// over nkt k-tiles whose fp32 output has rows_out rows of row_bytes (a tile
// row covers 256 of them).  The contraction kernel runs one workgroup per
// CU, so its time is estimated as the rounds of kCUs workgroups times the
// k-tiles each runs; cut k ranges add their partial outputs, written and
// then summed (2 P + 1 passes over those bytes).  Two forms are weighed:
//  - every tile cut into P slices (the launch has too few tiles for the CUs);
//  - the first tile rows whole, in as many full rounds as the tiles fill,
//    and only the last tile rows cut into P slices that fill the final
//    round instead of leaving most of its CUs idle.
// The least estimate is taken if it saves at least 1/16; each slice keeps at
// least 8 k-tiles.
KSplit k_split(int64_t tiles_m, int64_t tiles_n, int64_t nkt, int64_t rows_out, int64_t row_bytes, int esize) {
    constexpr int64_t kCUs = 256;                         // MI355X compute units
    const int64_t kt_ns = esize == 2 ? 2000 : 8000;       // one k-tile of one workgroup
    constexpr int64_t kBytesPerNs = 4000;                 // streaming rate of the partials
    const int64_t tiles = tiles_m * tiles_n;
    auto est = [&](int64_t P) {
        const int64_t per = (nkt + P - 1) / P, rounds = (tiles * P + kCUs - 1) / kCUs;
        return rounds * per * kt_ns + (P > 1 ? (2 * P + 1) * rows_out * row_bytes / kBytesPerNs : 0);
    };
    KSplit r{1, nkt, 0};
    const int64_t e1 = est(1);
    int64_t tb = e1;
    for (int64_t P = 2; P <= 8 && (nkt + P - 1) / P >= 8; ++P)
        if (est(P) < tb) r = KSplit{(int)P, 0, tiles_m}, tb = est(P);
    const int64_t full = tiles / kCUs;
    if (full >= 1) {
        const int64_t h = full * kCUs / tiles_n, t = tiles_m - h, tt = t * tiles_n;
        const int64_t P = t > 0 ? std::min<int64_t>(std::min<int64_t>(8, kCUs / tt), nkt / 8) : 0;
        if (P >= 2) {
            const int64_t per = (nkt + P - 1) / P;
            const int64_t tail_bytes = std::max<int64_t>(0, rows_out - 256 * h) * row_bytes;
            const int64_t e = (h * tiles_n + kCUs - 1) / kCUs * nkt * kt_ns + per * kt_ns +
                              (2 * P + 1) * tail_bytes / kBytesPerNs;
            if (e < tb) r = KSplit{(int)P, 0, t}, tb = e;
        }
    }
    if (tb > e1 - e1 / 16) r = KSplit{1, nkt, 0};
    if (r.P > 1) {
        r.nks = (nkt + r.P - 1) / r.P;
        r.P = (int)((nkt + r.nks - 1) / r.nks);
    }
    return r;
}

GatherFwdPlan gather_fwd_plan(int64_t N, int64_t I, int64_t O, int K, int D, int base) {
    GatherFwdPlan q;
    const int64_t ob = (O + kGatherFwdOutputs - 1) / kGatherFwdOutputs;
    // 256-row blocks of 1024 threads when they still make 64 or more blocks
    // (or when K is large, where staging dominates); 64-row blocks of 256
    // threads for small batches
    q.nt = ((N + 255) / 256 * ob >= 64 || K > 32) ? 1024 : 256;
    const int R = q.nt / 4;
    const int rw = ((D + 3) + 1) & ~1;                       // words of a span record
    const int64_t per_in = (int64_t)kGatherFwdOutputs * K + (base ? kGatherFwdOutputs : 0) + (int64_t)R * rw;
    // both chunk buffers within 150 KB (1024 threads, one block per CU) or
    // 64 KB (256 threads, two or more per CU); a chunk row of at most 256 / 128
    // coefficients per output, which the prefetch registers hold
    const int64_t budget = (q.nt == 1024 ? 150 * 1024 : 64 * 1024) / 4;
    const int lim = q.nt == 1024 ? 256 : 128;
    int64_t ic = std::min<int64_t>(8, budget / (2 * per_in));
    ic = std::min<int64_t>(ic, lim / K);
    q.ic = (int)std::max<int64_t>(ic, 1);
    q.lds = (size_t)(2 * q.ic * per_in * 4);
    q.rb = (N + R - 1) / R;
    q.ob = ob;
    // fewer blocks than CUs: split the inputs, at least 8 per slice
    const int64_t T = q.rb * q.ob;
    int64_t S = 1;
    if (N * I * O >= (int64_t(1) << 16) && T < 256)
        S = std::max<int64_t>(1, std::min<int64_t>((256 + T - 1) / T, (I + 7) / 8));
    q.is = (I + S - 1) / S;
    q.split = (int)((I + q.is - 1) / q.is);
    q.ws = q.split > 1 ? (size_t)round_up((int64_t)q.split * N * O * 8, 256) : 0;
    return q;
}

GatherBwdPlan gather_bwd_plan(int64_t N, int64_t I, int64_t O, int K, int base) {
    GatherBwdPlan q;
    const int64_t target = 256;                       // blocks that fill the CUs once
    const bool big = N * I * O >= (int64_t(1) << 16);
    // dx: the widest output chunk whose two buffers fit in 150 KB of LDS
    q.jc = 4;
    for (int jc : {16, 8}) {
        const int64_t floats = 2 * ((int64_t)kGatherDxRows * jc + (int64_t)kGatherDxInputs * K * (jc + 4) + kGatherDxInputs * (jc + 4));
        if (floats * 4 <= 150 * 1024) { q.jc = jc; break; }
    }
    q.lds_dx = (size_t)(2 * ((int64_t)kGatherDxRows * q.jc + (int64_t)kGatherDxInputs * K * (q.jc + 4) + kGatherDxInputs * (q.jc + 4)) * 4);
    q.rb = (N + kGatherDxRows - 1) / kGatherDxRows;
    q.ib = (I + kGatherDxInputs - 1) / kGatherDxInputs;
    int64_t sx = 1;
    if (big && q.rb * q.ib < target)
        sx = std::max<int64_t>(1, std::min((target + q.rb * q.ib - 1) / (q.rb * q.ib), (O + 4 * q.jc - 1) / (4 * q.jc)));
    q.js = ((O + sx - 1) / sx + q.jc - 1) / q.jc * q.jc;
    q.sx = (int)((O + q.js - 1) / q.js);
    // dC: KMAX register sums per lane and output; two outputs per lane when
    // the sums of both fit 1024-thread blocks (KMAX <= 32) and the layer has
    // more than 64 outputs, one otherwise; waves of one block share a dy
    // chunk; 512-thread blocks where the sums need more than the 128
    // registers of 1024 threads
    q.kmax = K <= 16 ? 16 : K <= 32 ? 32 : K <= 64 ? 64 : 132;    // K <= 125 + 5
    q.opl = q.kmax <= 32 && O > 64 ? 2 : 1;
    q.nt_dc = q.kmax * q.opl <= 64 ? 1024 : 512;
    const int nw = q.nt_dc / 64;
    q.ibn = (I + nw - 1) / nw;
    q.ob = (O + 64 * q.opl - 1) / (64 * q.opl);
    q.lds_dc = (size_t)(2 * (64 * 64 * q.opl + nw * 64 * kGatherDcRecord) * 4);
    int64_t sc = 1;
    if (big && q.ibn * q.ob < target)
        sc = std::max<int64_t>(1, std::min((target + q.ibn * q.ob - 1) / (q.ibn * q.ob), (N + 127) / 128));
    q.rs = std::max<int64_t>(64, ((N + sc - 1) / sc + 63) / 64 * 64);
    q.sc = (int)std::max<int64_t>(1, (N + q.rs - 1) / q.rs);
    // workspace: dx partials, then dC and dW_base partials
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (size_t)round_up((int64_t)bytes, 256);
        return o;
    };
    q.off_dxp = q.sx > 1 ? take((size_t)q.sx * N * I * 4) : 0;
    q.off_dcp = q.sc > 1 ? take((size_t)q.sc * O * I * K * 4) : 0;
    q.off_dwp = q.sc > 1 && base ? take((size_t)q.sc * O * I * 4) : 0;
    q.ws = off;
    return q;
}

// Row chunks.  The forward aims at 2048 blocks (8 per CU, one round).  The
// backward aims at 1024 (4 per CU) and gives every chunk at least
// max(64, 24 K) rows, so that the partials (K floats per channel per chunk,
// written and read back) stay within about 1/30 of the traffic of x, dy and
// dx.  Chunks are whole multiples of the rows a block's waves take per step.
GroupPlan grouped_plan(int64_t N, int64_t I, int K) {
    GroupPlan gp;
    gp.xb = (I + kGroupChannels - 1) / kGroupChannels;
    auto chunk = [&](int64_t blocks, int64_t rmin, int64_t step) {
        const int64_t gy = std::max<int64_t>(1, blocks / gp.xb);
        return round_up(std::max<int64_t>(rmin, (N + gy - 1) / gy), step);
    };
    gp.rows_fwd = chunk(2048, 1, kGroupWaves * kGroupRowsFwd);
    gp.rows_bwd = chunk(1024, std::max<int64_t>(64, 24 * (int64_t)K), kGroupWaves * kGroupRowsBwd);
    gp.gy_fwd = (N + gp.rows_fwd - 1) / gp.rows_fwd;
    gp.gy_bwd = (N + gp.rows_bwd - 1) / gp.rows_bwd;
    gp.part_floats = gp.gy_bwd * K * I;
    gp.red_floats = (int64_t)K * I;
    return gp;
}

}  // namespace kan
