// Dense-basis KAN contractions on the gfx950 matrix cores.
//
// With C' = [C | W_base] per input (Kb = G+3+has_base columns per input) and
// Phi'(x) the dense basis row [B_0(x_i) .. B_{G+2}(x_i), silu(x_i)] per input,
// the three contractions of a training step are GEMMs over generated or
// packed operands:
//
//   forward  y   [N, O]      = Phi'[N, I*Kb]  . C'^T          (k = (i, m))
//   dx       P   [N, I*Kb]   = dy [N, O]      . C'            (k = j), then
//            dx[b, i] = sum_m P[b, i, m] B'_m(x[b, i]) + P[b, i, K] silu'(x[b, i])
//   dC, dW   dC' [O, I*Kb]   = dy^T [O, N]    . Phi'[N, I*Kb] (k = b)
//
// Phi' is generated tile by tile in LDS from x (span, 4 pieces, silu: InKAN
// project page, "Why InKAN?") and is never written to memory (UKAN / warpKAN
// abstract: the memory saving of not materialising the basis).  The dC'
// reduction over the batch is owned by one workgroup per output tile and runs
// in a fixed order without atomics (FlashKAT abstract: atomic gradient
// accumulation and memory stalls are what slow the backward pass).
//
// Tiling: 256 x 256 output tile per workgroup of 8 waves (4 x 2 waves of
// 64 x 128 = 2 x 4 MFMA blocks of 32 x 32, two waves per SIMD), k-tiles of
// 128 bytes per row (64 bf16 / 32 float), two LDS stages of A and B with a
// 144-byte row pitch; global loads run two k-tiles ahead of the MFMAs.
// bf16 uses v_mfma_f32_32x32x16_bf16, float uses v_mfma_f32_32x32x2_f32;
// both accumulate in float32.  The 32 x 32 blocks keep each accumulator in
// one 16-register tuple, which the register allocator leaves in place (16 x
// 16 blocks made it shuttle accumulators between register files every
// k-tile).  Each lane reads 16 contiguous bytes of k per fragment row, so A
// and B share one lane -> k assignment and the k order inside a step does
// not matter.
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "kan_internal.h"
#include "kan_sparse.h"

namespace kan {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes in 4 registers
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x8 make_u32x8(const uint4& lo, const uint4& hi) {
    u32x8 v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
}

constexpr int PITCH = 144;                     // bytes per LDS tile row (128 data + 16 pad)
constexpr int TILE_BYTES = 256 * PITCH;        // one 256-row operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // A + B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;     // two stages: 147456 bytes
constexpr int DX_PITCH = 260;                  // floats per row of the dx epilogue staging
constexpr int BLOCK_BYTES = 256 * 128;         // one packed k-tile of one 256-row tile

template <typename TS> struct Traits;
template <> struct Traits<uint16_t> {          // bf16 storage
    static constexpr int ES = 2;
    static constexpr int BK = 64;
    // one 32-byte k-step per row: 16 bf16
    __device__ static void mma(f32x16& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    // v_cvt_pk_bf16_f32: round to nearest even
    __device__ static void put(char* p, float v) {
        *reinterpret_cast<uint16_t*>(p) = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
    // A pair's 4 basis values and silu value in storage form: two values per
    // conversion; store<r> writes value r (4: silu) from its half.
    struct Vals { uint32_t p01, p23, ps; };
    // v_cvt_pk_bf16_f32 of two values (left to itself the compiler converts
    // each value on its own and stores both halves from separate registers)
    __device__ static uint32_t pk(float a, float b) {
        uint32_t r;
        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
        return r;
    }
    __device__ static Vals vals(float u, float silu_x) {
        float b0, b1, b2, b3;
        pieces_fast(u, b0, b1, b2, b3);
        return Vals{pk(b0, b1), pk(b2, b3), pk(silu_x, 0.0f)};
    }
    template <int r>
    __device__ static void store(char* p, const Vals& v) {
        const uint32_t w = r < 2 ? v.p01 : r < 4 ? v.p23 : v.ps;
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)((r & 1) ? (w >> 16) : w);
    }
};
template <> struct Traits<float> {
    static constexpr int ES = 4;
    static constexpr int BK = 32;
    // one 32-byte k-step per row: 8 floats, lane half h holds k = 4h .. 4h+3;
    // MFMA e pairs k = e (lanes 0-31) with k = 4 + e (lanes 32-63)
    __device__ static void mma(f32x16& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
    __device__ static void put(char* p, float v) { *reinterpret_cast<float*>(p) = v; }
    struct Vals { float v[5]; };
    __device__ static Vals vals(float u, float silu_x) {
        Vals r;
        pieces(u, r.v[0], r.v[1], r.v[2], r.v[3]);
        r.v[4] = silu_x;
        return r;
    }
    template <int r>
    __device__ static void store(char* p, const Vals& v) { *reinterpret_cast<float*>(p) = v.v[r]; }
};

// x as loaded into a generator slot: the stored bits in a 32-bit register
// (bf16 zero-extended), turned into a float where it is used.
__device__ __forceinline__ uint32_t raw_bits(const float* p, int64_t i) { return __float_as_uint(p[i]); }
__device__ __forceinline__ uint32_t raw_bits(const uint16_t* p, int64_t i) { return p[i]; }
template <typename TS> __device__ __forceinline__ float raw_to_float(uint32_t w);
template <> __device__ __forceinline__ float raw_to_float<float>(uint32_t w) { return __uint_as_float(w); }
template <> __device__ __forceinline__ float raw_to_float<uint16_t>(uint32_t w) { return __uint_as_float(w << 16); }

// Calls f(std::integral_constant<int, I>()) for I = B .. E-1, so that the
// index is a constant expression inside f.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}

struct GemmArgs {
    int tiles_m, tiles_n, nkt, group_m;
    const char* a;       // loaded A operand (blocked, see LoadOp), or null
    int64_t a_tstride;   // bytes per 256-row tile: k-tiles * BLOCK_BYTES
    const char* b;       // loaded B operand, or null
    int64_t b_tstride;
    const void* x;       // generator input x [N, I]
    GridK g;
    int N, I, O, K, Kb, base;
    int xI;              // x row width: I, or 2P for the pairs of the 2-D layer
    int deg;             // spline degree (the K-variant operands; the cubic ones assume 3)
    int64_t IKb;
    float* out0;         // y, dx or dC
    float* out1;         // dW_base, or the dx partial sums
    // k-split of the last `tail` tile rows (0: none): slice s of such a tile
    // runs k-tiles [nks s, min(nkt, nks (s + 1))) and writes its epilogue
    // output to part0 + s * ostride0 - oshift0 in place of out0 (part1,
    // ostride1, oshift1 in place of out1): the partial arrays hold the tail
    // rows only, and oshift* is the output offset of the first tail row
    int tail, nks;
    float* part0;
    float* part1;
    int64_t ostride0, ostride1, oshift0, oshift1;
};

// Tile order: workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Give every XCD a contiguous range of tile ids, and walk
// ids in groups of `group_m` tile rows so that the workgroups resident on one
// XCD share their B tiles (and their A tiles across the group).  The grid
// holds the whole tiles of the first tiles_m - tail tile rows, then slice 0
// of every tail tile, slice 1, and so on; returns the slice.
__device__ __forceinline__ int tile_coords(const GemmArgs& a, int& tm, int& tn) {
    int bid = blockIdx.x, slice = 0, row0 = 0, rows = a.tiles_m - a.tail;
    const int head = rows * a.tiles_n;
    if (bid >= head) {
        bid -= head;
        row0 = rows;
        rows = a.tail;
        slice = bid / (rows * a.tiles_n);
        bid -= slice * rows * a.tiles_n;
    }
    const int total = rows * a.tiles_n;
    const int nfull = total / 8, rem = total % 8;
    const int xcd = bid % 8, slot = bid / 8;
    const int id = xcd * nfull + min(xcd, rem) + slot;
    const int per_group = a.group_m * a.tiles_n;
    const int grp = id / per_group;
    const int first_m = grp * a.group_m;
    const int gm = min(rows - first_m, a.group_m);
    const int r = id - grp * per_group;
    tm = row0 + first_m + r % gm;
    tn = r / gm;
    return slice;
}

// ---- operands ----
// Every operand holds DEPTH = 2 register slots; the k-loop names a slot by a
// compile-time index SL.  Hooks:
//   fetch<SL>(kt)             start the global loads of k-tile kt into slot SL
//                             (a copied operand: the tile itself; a generated
//                             one: the x values it needs)
//   part<SL, RF>(S, kt, ktn, p)  write part p (of NPART) of k-tile kt from
//                             slot SL into LDS tile S, then (if RF) start
//                             refilling what that part freed with k-tile
//                             ktn = kt + DEPTH
// The parts are spread over the MFMA k-steps of the tile being multiplied, so
// LDS stores, generator arithmetic and load issue overlap the matrix cores
// instead of forming a phase of their own before each barrier.  A part's
// loads are issued two k-tiles before the part is stored, and no slot is
// ever copied (a register copy out of a slot whose loads are in flight would
// wait for them).  The workgroup has 8 waves (2 per SIMD), arranged 4 x 2
// over the 256 x 256 tile; wave w owns rows 64 (w / 2) .. +64 and columns
// 128 (w % 2) .. +128.
constexpr int NTHR = 512;

// Operand copied from a blocked packed array: k-tile kt of 256-row tile T is
// one contiguous block of 256 rows x 128 bytes at T * tstride + kt *
// BLOCK_BYTES.  (Row-major operands put the 256 rows of a k-tile kilobytes
// apart, one page each, and loading them cost a quarter of the run time.)
// Part q: thread t loads bytes 8192 q + 16 t of the block, i.e. row
// 64 q + t / 8, 16-byte chunk t % 8, so one wave instruction reads 1 KB in
// order; the part goes through registers into LDS.
struct LoadOp {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int NPART = 4;
    static constexpr int DEPTH = 2;
    const char* base;    // this thread's 16 bytes of k-tile 0 of the tile
    u32x4 v[2][4];
    __device__ LoadOp(const char* p, int64_t tile, int64_t tstride)
        : base(p + tile * tstride + threadIdx.x * 16) {}
    template <int SL>
    __device__ __forceinline__ void load(int kt, int q) {
        v[SL][q] = *reinterpret_cast<const u32x4*>(base + (int64_t)kt * BLOCK_BYTES + q * 8192);
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs&, int kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) load<SL>(kt, q);
    }
    template <int SL, bool RF, int q>
    __device__ __forceinline__ void part(const GemmArgs&, char* S, int, int ktn) {
        const int t = threadIdx.x, c = t & 7, r = t >> 3;
        *reinterpret_cast<u32x4*>(S + (r + 64 * q) * PITCH + c * 16) = v[SL][q];
        if (RF) load<SL>(ktn, q);
    }
};
struct LoadA : LoadOp {                // tile tm of A
    __device__ LoadA(const GemmArgs& a, int tm, int) : LoadOp(a.a, tm, a.a_tstride) {}
};
struct LoadB : LoadOp {                // tile tn of B
    __device__ LoadB(const GemmArgs& a, int, int tn) : LoadOp(a.b, tn, a.b_tstride) {}
};

// Forward A operand Phi'[b, (i, m)].  The (row, input) pairs of a k-tile are
// dealt to all 512 threads with the NIN inputs of one row in NIN adjacent
// lanes (NIN a power of two dividing the wave), so one load instruction
// touches 64 / NIN rows of x rather than 64.  The lanes of a row zero-fill it
// and then scatter its <= 4 spline values and silu value per input; they are
// in one wave, whose LDS writes land in program order, so no barrier is
// needed between the two.  x loads are clamped in bounds and writes that fall
// outside the tile go to the row's 16 pad bytes, which no fragment read
// touches: the generator has no divergent branches.  Rows past N are
// generated from a clamped row and never stored by the epilogue.
template <typename TS, int NIN>
struct GenA {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPT = 256 * NIN / NTHR;       // pairs per thread
    static constexpr int NPART = PPT;                  // part j: pair j (its row)
    static constexpr int DEPTH = 2;                    // two slots of x values
    static constexpr int RSTEP = NTHR / NIN;           // rows between a thread's pairs
    static_assert(NIN >= 2 && (NIN & (NIN - 1)) == 0 && NIN <= 32, "NIN: power of two");
    const TS* x;
    int q, row0;
    int64_t xrow[PPT];
    float xs[2][PPT];    // slots: x values of this lane's pairs
    int is[2];           // slots: this lane's input
    __device__ GenA(const GemmArgs& a, int tm, int) {
        x = static_cast<const TS*>(a.x);
        q = threadIdx.x % NIN;
        row0 = threadIdx.x / NIN;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            xrow[j] = (int64_t)min(tm * 256 + row0 + RSTEP * j, a.N - 1) * a.I;
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
        is[SL] = (unsigned)(kt * BK) / (unsigned)a.Kb + q;
        const int i = min(is[SL], a.I - 1);
#pragma unroll
        for (int j = 0; j < PPT; ++j) xs[SL][j] = load_f(x, xrow[j] + i);
    }
    // Pair j: the NIN lanes of its row clear the row's 8 chunks of 16 bytes,
    // then each scatters its input's <= 4 spline values and silu value.
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* row = S + (row0 + RSTEP * j) * PITCH;
#pragma unroll
        for (int c = 0; c < (8 + NIN - 1) / NIN; ++c) {
            const int chunk = q * ((8 + NIN - 1) / NIN) + c;
            *reinterpret_cast<uint4*>(row + (chunk < 8 ? 16 * chunk : BK * ES)) = make_uint4(0, 0, 0, 0);
        }
        // This lane's input i covers tile columns cb .. cb + Kb - 1; spline
        // index m is written when lo <= m < lo + n (inside [0, K) and inside
        // the tile), the silu column when vs.  Both hold for the whole k-tile.
        const int i = is[SL];
        const int cb = i * a.Kb - kt * BK;
        const int lo = max(0, -cb);
        const int n = i < a.I ? max(0, min(a.K, BK - cb) - lo) : 0;
        const int cs = cb + a.K;
        const bool vs = (a.base != 0) & (i < a.I) & ((unsigned)cs < (unsigned)BK);
        const float xv = xs[SL][j];
        float u;
        const int s = span_u(xv, a.g, u);
        const typename Traits<TS>::Vals val = Traits<TS>::vals(u, silu(xv));
        // value r goes to column cb + s - 3 + r; a rejected one to the pad
        char* first = row + (cb + s - 3) * ES;
        char* pad = row + BK * ES;
        static_for<0, 4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const bool v = (unsigned)(s - 3 - lo + r) < (unsigned)n;
            Traits<TS>::template store<r>((v ? first : pad) + r * ES, val);
        });
        Traits<TS>::template store<4>(vs ? row + cs * ES : pad, val);
        if constexpr (RF && j == NPART - 1) fetch<SL>(a, ktn);
    }
};

// Forward A operand of a bf16 layer from the truncated-power form (FlashKAN
// project page: a cubic B-spline is a combination of five shifted truncated
// cubes of the normalised coordinate, clamped to [0, 4]).  Every tile column
// (i, m) is evaluated on its own from u = x / h + (shift - m): there is no
// span, no zero fill and no scatter.  Pairs and lanes as in GenA (NIN
// adjacent lanes per row, one input each); a lane writes every tile column of
// its input, the silu column included, and zeros for inputs past the last
// one, so the tile is complete without a fill.  Columns whose u lies outside
// (0, 4) come out exactly 0 (all terms vanish, or cancel exactly at u = 4).
template <int NIN>
struct GenT {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<uint16_t>::BK;
    static constexpr int ES = Traits<uint16_t>::ES;
    static constexpr int PPT = 256 * NIN / NTHR;       // pairs per thread
    static constexpr int NPART = PPT;                  // part j: pair j (its row)
    static constexpr int DEPTH = 2;                    // two slots of x values
    static constexpr int RSTEP = NTHR / NIN;           // rows between a thread's pairs
    static_assert(NIN >= 2 && (NIN & (NIN - 1)) == 0 && NIN <= 32, "NIN: power of two");
    const uint16_t* x;
    int q, row0;
    int64_t xrow[PPT];
    float xs[2][PPT];
    int is[2];
    __device__ GenT(const GemmArgs& a, int tm, int) {
        x = static_cast<const uint16_t*>(a.x);
        q = threadIdx.x % NIN;
        row0 = threadIdx.x / NIN;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            xrow[j] = (int64_t)min(tm * 256 + row0 + RSTEP * j, a.N - 1) * a.I;
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
        is[SL] = (unsigned)(kt * BK) / (unsigned)a.Kb + q;
        const int i = min(is[SL], a.I - 1);
#pragma unroll
        for (int j = 0; j < PPT; ++j) xs[SL][j] = load_f(x, xrow[j] + i);
    }
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* row = S + (row0 + RSTEP * j) * PITCH;
        const int i = is[SL];
        const int cb = i * a.Kb - kt * BK;             // tile column of (i, 0)
        const bool live = i < a.I;
        const float xv = xs[SL][j];
        const float sx = live && a.base ? silu(xv) : 0.0f;
        const float u0 = __builtin_fmaf(xv, a.g.scale, a.g.shift);
        char* pad = row + BK * ES;
        // a trip count uniform over the block: columns outside the tile go
        // to the row's pad bytes
#pragma nounroll
        for (int m = 0; m < a.Kb; ++m) {
            const int c = cb + m;
            float b = sx, d;
            tp_basis(u0 - (float)m, a.g.scale, b, d);
            if (m >= a.K) b = sx;
            Traits<uint16_t>::put((unsigned)c < (unsigned)BK ? row + c * ES : pad, live ? b : 0.0f);
        }
        if constexpr (RF && j == NPART - 1) fetch<SL>(a, ktn);
    }
};

// dC B operand Phi'^T[(i, m), b]: tile rows are the 256 packed columns
// n0 .. n0+255 of Phi', k runs over the batch.  Wave w owns the NQW tile
// inputs w NQW .. w NQW + NQW - 1: it zero-fills their tile rows and then
// scatters their non-zeros, in program order, so no barrier is needed.  The
// wave's (row b, input) pairs run input-fastest over its lanes, so one x load
// instruction touches 64 / NQW rows of x.  ZR = ceil(Kb / 8) zero-fill
// instructions per input; writes outside the tile go to the pad bytes of
// row 0.
template <typename TS, int NQW, int ZR>
struct GenB {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPL = BK * NQW / 64;            // pairs per lane
    static constexpr int NPART = 1 + PPL;                // zero fill, then pair by pair
    static constexpr int DEPTH = 2;                      // two slots of x values
    static_assert(BK * NQW % 64 == 0, "whole pairs per lane");
    const TS* x;
    int n0, i0, wave, lane;
    int bl[PPL], il[PPL];
    // per pair: byte offset of (row of (i, m = 0), column b) in the tile (row
    // may be negative), valid spline index range [lo, lo + n), and the silu
    // value's offset (the pad of row 0 when it has no place in the tile)
    int off[PPL], lo[PPL], cnt[PPL], soff[PPL];
    float xs[2][PPL];    // slots: x values of this lane's pairs
    __device__ GenB(const GemmArgs& a, int, int tn) {
        x = static_cast<const TS*>(a.x);
        n0 = tn * 256;
        lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
        i0 = (unsigned)n0 / (unsigned)a.Kb + wave * NQW;  // first input of this wave
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int pp = lane + 64 * j;
            bl[j] = pp / NQW;
            il[j] = pp % NQW;
            const int i = i0 + il[j];
            const int rb = i * a.Kb - n0;                 // tile row of (i, m = 0)
            off[j] = rb * PITCH + bl[j] * ES;
            lo[j] = max(0, -rb);
            cnt[j] = i < a.I ? max(0, min(a.K, 256 - rb) - lo[j]) : 0;
            const int rs = rb + a.K;
            soff[j] = (a.base != 0) & (i < a.I) & ((unsigned)rs < 256u) ? rs * PITCH + bl[j] * ES : 128;
        }
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int64_t brow = (int64_t)min(kt * BK + bl[j], a.N - 1) * a.I;
            xs[SL][j] = load_f(x, brow + min(i0 + il[j], a.I - 1));
        }
    }
    template <int SL, bool RF, int p>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        if constexpr (p == 0) {
            // zero the rows of this wave's inputs: 8 rows of 128 bytes per instruction
#pragma unroll
            for (int e = 0; e < NQW; ++e) {
                const int rb = (i0 + e) * a.Kb - n0;
#pragma unroll
                for (int z = 0; z < ZR; ++z) {
                    const int rr = 8 * z + (lane >> 3);
                    const int row = rb + rr;
                    const bool v = (rr < a.Kb) & (row >= 0) & (row < 256);
                    *reinterpret_cast<uint4*>(v ? S + row * PITCH + (lane & 7) * 16 : S + 128) =
                        make_uint4(0, 0, 0, 0);
                }
            }
            return;
        } else {
        constexpr int j = p - 1;
        // Batch rows past N are generated from a clamped row: dy^T is zero
        // there, so they add nothing.
        const float xv = xs[SL][j];
        float u;
        const int s = min(span_u(xv, a.g, u), a.K + 3);   // larger spans hold no index < K
        const typename Traits<TS>::Vals val = Traits<TS>::vals(u, silu(xv));
        // value r goes to tile row rb + s - 3 + r; a rejected one to the pad
        // of row r
        const int first = off[j] + (s - 3) * PITCH;
        static_for<0, 4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const bool v = (unsigned)(s - 3 - lo[j] + r) < (unsigned)cnt[j];
            Traits<TS>::template store<r>(S + (v ? first : 128) + r * PITCH, val);
        });
        Traits<TS>::template store<4>(S + soff[j], val);
        if constexpr (RF && p == NPART - 1) fetch<SL>(a, ktn);
        }
    }
};

// ---- 2-D tensor-product layer: operands of the pairs ----
// A pair p = (x[b, 2p], x[b, 2p+1]) owns Kb = K1^2 columns p Kb + m K1 + n
// (K1 = G + 3); of them the 16 with m = s1-3+r, n = s2-3+q (r, q < 4, s1, s2
// the spans of the two inputs) hold the products b_r(u1) b_q(u2), the rest
// are zero.  Spans past K1 + 3 hold no index < K1 and are clamped there, so
// the column arithmetic stays small.
__device__ __forceinline__ void pair_pieces(float x1, float x2, const GridK& g, int& s1, int& s2, float w1[4],
                                            float w2[4]) {
    const int K1 = g.G + 3;
    float u1, u2;
    s1 = min(span_u(x1, g, u1), K1 + 3);
    s2 = min(span_u(x2, g, u2), K1 + 3);
    pieces(u1, w1[0], w1[1], w1[2], w1[3]);
    pieces(u2, w2[0], w2[1], w2[2], w2[3]);
}

// Forward A operand of the 2-D layer: GenA with pairs for inputs.  The NIN
// lanes of a row clear it and scatter their pair's <= 16 products (a column
// outside the k-tile, or a product with m or n outside [0, K1), goes to the
// row's pad bytes).
template <typename TS, int NIN>
struct GenA2 {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPT = 256 * NIN / NTHR;       // (row, pair) items per thread
    static constexpr int NPART = PPT;
    static constexpr int DEPTH = 2;
    static constexpr int RSTEP = NTHR / NIN;
    static_assert(NIN >= 2 && (NIN & (NIN - 1)) == 0 && NIN <= 32, "NIN: power of two");
    const TS* x;
    int q, row0;
    int64_t xrow[PPT];
    float x1s[2][PPT], x2s[2][PPT];
    int ps[2];
    __device__ GenA2(const GemmArgs& a, int tm, int) {
        x = static_cast<const TS*>(a.x);
        q = threadIdx.x % NIN;
        row0 = threadIdx.x / NIN;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            xrow[j] = (int64_t)min(tm * 256 + row0 + RSTEP * j, a.N - 1) * a.xI;
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
        ps[SL] = (unsigned)(kt * BK) / (unsigned)a.Kb + q;
        const int p = min(ps[SL], a.I - 1);
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            x1s[SL][j] = load_f(x, xrow[j] + 2 * p);
            x2s[SL][j] = load_f(x, xrow[j] + 2 * p + 1);
        }
    }
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* row = S + (row0 + RSTEP * j) * PITCH;
#pragma unroll
        for (int c = 0; c < (8 + NIN - 1) / NIN; ++c) {
            const int chunk = q * ((8 + NIN - 1) / NIN) + c;
            *reinterpret_cast<uint4*>(row + (chunk < 8 ? 16 * chunk : BK * ES)) = make_uint4(0, 0, 0, 0);
        }
        const int K1 = a.g.G + 3;
        const int p = ps[SL];
        const int cb = p * a.Kb - kt * BK;               // tile column of (p, 0, 0)
        const bool live = p < a.I;
        int s1, s2;
        float w1[4], w2[4];
        pair_pieces(x1s[SL][j], x2s[SL][j], a.g, s1, s2, w1, w2);
        char* pad = row + BK * ES;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = s1 - 3 + r;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = s2 - 3 + qq, c = cb + m * K1 + n;
                const bool v = live & ((unsigned)m < (unsigned)K1) & ((unsigned)n < (unsigned)K1) &
                               ((unsigned)c < (unsigned)BK);
                Traits<TS>::put(v ? row + c * ES : pad, w1[r] * w2[qq]);
            }
        }
        if constexpr (RF && j == NPART - 1) fetch<SL>(a, ktn);
    }
};

// dC B operand of the 2-D layer: GenB with pairs for inputs.  Tile rows are
// the packed columns n0 .. n0+255 (pair, m, n); k runs over the batch.  Wave
// w clears the rows of its NQW pairs, then each (row b, pair) scatters its
// <= 16 products into column b (rejected ones to pad bytes).
template <typename TS, int NQW, int ZR>
struct GenB2 {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPL = BK * NQW / 64;            // (row, pair) items per lane
    static constexpr int NPART = 1 + PPL;
    static constexpr int DEPTH = 2;
    static_assert(BK * NQW % 64 == 0, "whole items per lane");
    const TS* x;
    int n0, i0, wave, lane;
    int bl[PPL], il[PPL], rb[PPL];
    float x1s[2][PPL], x2s[2][PPL];
    __device__ GenB2(const GemmArgs& a, int, int tn) {
        x = static_cast<const TS*>(a.x);
        n0 = tn * 256;
        lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
        i0 = (unsigned)n0 / (unsigned)a.Kb + wave * NQW;  // first pair of this wave
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int pp = lane + 64 * j;
            bl[j] = pp / NQW;
            il[j] = pp % NQW;
            const int p = i0 + il[j];
            // tile row of (p, 0, 0); a pair past the last one gets a row that
            // no product can reach
            rb[j] = p < a.I ? p * a.Kb - n0 : 1 << 20;
        }
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int64_t brow = (int64_t)min(kt * BK + bl[j], a.N - 1) * a.xI;
            const int p = min(i0 + il[j], a.I - 1);
            x1s[SL][j] = load_f(x, brow + 2 * p);
            x2s[SL][j] = load_f(x, brow + 2 * p + 1);
        }
    }
    template <int SL, bool RF, int pi>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        if constexpr (pi == 0) {
#pragma unroll
            for (int e = 0; e < NQW; ++e) {
                const int r0 = (i0 + e) * a.Kb - n0;
#pragma unroll
                for (int z = 0; z < ZR; ++z) {
                    const int rr = 8 * z + (lane >> 3);
                    const int row = r0 + rr;
                    const bool v = (rr < a.Kb) & (row >= 0) & (row < 256);
                    *reinterpret_cast<uint4*>(v ? S + row * PITCH + (lane & 7) * 16 : S + 128) =
                        make_uint4(0, 0, 0, 0);
                }
            }
            return;
        } else {
        constexpr int j = pi - 1;
        // batch rows past N come from a clamped row; dy^T is zero there
        const int K1 = a.g.G + 3;
        int s1, s2;
        float w1[4], w2[4];
        pair_pieces(x1s[SL][j], x2s[SL][j], a.g, s1, s2, w1, w2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = s1 - 3 + r;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = s2 - 3 + qq, t = rb[j] + m * K1 + n;
                const bool v = ((unsigned)m < (unsigned)K1) & ((unsigned)n < (unsigned)K1) &
                               ((unsigned)t < 256u);
                Traits<TS>::put(S + (v ? t * PITCH + bl[j] * ES : 128 + (4 * r + qq) * PITCH),
                                w1[r] * w2[qq]);
            }
        }
        if constexpr (RF && pi == NPART - 1) fetch<SL>(a, ktn);
        }
    }
};

// ---- layers of spline degree D != 3: the same operands with D + 1 values ----
// GenAK / GenBK / EpiDXK are GenA / GenB / EpiDX with the D + 1 non-zero
// basis values (and derivatives) of local_basis_rt in place of the 4 cubic
// pieces; a.K = G + D and a.g places t_0 = lo - D h.  Spans past K + D hold
// no index < K and are clamped there.
template <typename TS, int NIN>
struct GenAK {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPT = 256 * NIN / NTHR;
    static constexpr int NPART = PPT;
    static constexpr int DEPTH = 2;
    static constexpr int RSTEP = NTHR / NIN;
    static_assert(NIN >= 2 && (NIN & (NIN - 1)) == 0 && NIN <= 32, "NIN: power of two");
    const TS* x;
    int q, row0;
    int64_t xrow[PPT];
    float xs[2][PPT];
    int is[2];
    __device__ GenAK(const GemmArgs& a, int tm, int) {
        x = static_cast<const TS*>(a.x);
        q = threadIdx.x % NIN;
        row0 = threadIdx.x / NIN;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            xrow[j] = (int64_t)min(tm * 256 + row0 + RSTEP * j, a.N - 1) * a.I;
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
        is[SL] = (unsigned)(kt * BK) / (unsigned)a.Kb + q;
        const int i = min(is[SL], a.I - 1);
#pragma unroll
        for (int j = 0; j < PPT; ++j) xs[SL][j] = load_f(x, xrow[j] + i);
    }
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* row = S + (row0 + RSTEP * j) * PITCH;
#pragma unroll
        for (int c = 0; c < (8 + NIN - 1) / NIN; ++c) {
            const int chunk = q * ((8 + NIN - 1) / NIN) + c;
            *reinterpret_cast<uint4*>(row + (chunk < 8 ? 16 * chunk : BK * ES)) = make_uint4(0, 0, 0, 0);
        }
        const int D = a.deg;
        const int i = is[SL];
        const int cb = i * a.Kb - kt * BK;
        const int lo = max(0, -cb);
        const int n = i < a.I ? max(0, min(a.K, BK - cb) - lo) : 0;
        const int cs = cb + a.K;
        const bool vs = (a.base != 0) & (i < a.I) & ((unsigned)cs < (unsigned)BK);
        const float xv = xs[SL][j];
        float u;
        const int s = min(span_u(xv, a.g, u), a.K + D);
        float b[6], dd[6];
        local_basis_rt(u, a.g.scale, D, b, dd);
        char* pad = row + BK * ES;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const bool v = (r <= D) & ((unsigned)(s - D - lo + r) < (unsigned)n);
            Traits<TS>::put(v ? row + (cb + s - D + r) * ES : pad, b[r]);
        }
        Traits<TS>::put(vs ? row + cs * ES : pad, silu(xv));
        if constexpr (RF && j == NPART - 1) fetch<SL>(a, ktn);
    }
};

template <typename TS, int NQW, int ZR>
struct GenBK {
    static constexpr bool SPARSE = false;
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    static constexpr int BK = Traits<TS>::BK;
    static constexpr int ES = Traits<TS>::ES;
    static constexpr int PPL = BK * NQW / 64;
    static constexpr int NPART = 1 + PPL;
    static constexpr int DEPTH = 2;
    static_assert(BK * NQW % 64 == 0, "whole pairs per lane");
    const TS* x;
    int n0, i0, wave, lane;
    int bl[PPL], il[PPL];
    int off[PPL], lo[PPL], cnt[PPL], soff[PPL];
    float xs[2][PPL];
    __device__ GenBK(const GemmArgs& a, int, int tn) {
        x = static_cast<const TS*>(a.x);
        n0 = tn * 256;
        lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
        i0 = (unsigned)n0 / (unsigned)a.Kb + wave * NQW;
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int pp = lane + 64 * j;
            bl[j] = pp / NQW;
            il[j] = pp % NQW;
            const int i = i0 + il[j];
            const int rb = i * a.Kb - n0;
            off[j] = rb * PITCH + bl[j] * ES;
            lo[j] = max(0, -rb);
            cnt[j] = i < a.I ? max(0, min(a.K, 256 - rb) - lo[j]) : 0;
            const int rs = rb + a.K;
            soff[j] = ((a.base != 0) & (i < a.I) & ((unsigned)rs < 256u)) ? rs * PITCH + bl[j] * ES : 128;
        }
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const int64_t brow = (int64_t)min(kt * BK + bl[j], a.N - 1) * a.I;
            xs[SL][j] = load_f(x, brow + min(i0 + il[j], a.I - 1));
        }
    }
    template <int SL, bool RF, int p>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        if constexpr (p == 0) {
#pragma unroll
            for (int e = 0; e < NQW; ++e) {
                const int rb = (i0 + e) * a.Kb - n0;
#pragma unroll
                for (int z = 0; z < ZR; ++z) {
                    const int rr = 8 * z + (lane >> 3);
                    const int row = rb + rr;
                    const bool v = (rr < a.Kb) & (row >= 0) & (row < 256);
                    *reinterpret_cast<uint4*>(v ? S + row * PITCH + (lane & 7) * 16 : S + 128) =
                        make_uint4(0, 0, 0, 0);
                }
            }
            return;
        } else {
        constexpr int j = p - 1;
        const int D = a.deg;
        const float xv = xs[SL][j];
        float u;
        const int s = min(span_u(xv, a.g, u), a.K + D);
        float b[6], dd[6];
        local_basis_rt(u, a.g.scale, D, b, dd);
        const int first = off[j] + (s - D) * PITCH;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const bool v = (r <= D) & ((unsigned)(s - D - lo[j] + r) < (unsigned)cnt[j]);
            Traits<TS>::put(S + (v ? first + r * PITCH : 128 + r * PITCH), b[r]);
        }
        Traits<TS>::put(S + soff[j], silu(xv));
        if constexpr (RF && p == NPART - 1) fetch<SL>(a, ktn);
        }
    }
};

// Forward A operand in 2:4 structured-sparse form (bf16 only), in the column
// order of kan_sparse.h; the coefficient operand is packed in the same order
// (pack_fwd_sparse).
//
// A k-tile is 64 logical columns = 16 groups.  LDS row (PITCH bytes): group G
// in [-8, 24) keeps its two values at byte 4 (G + 8); the tile's groups 0..15
// are bytes 32..95, the rest is margin that inputs straddling the tile write
// and no fragment reads.  The index nibbles of groups G, G + 1 (G even) are
// byte 128 + ((G + 16) / 2) % 16, so groups 0..15 are bytes 136..143.
//
// Each pair builds its input's whole block of NG dwords in registers and
// writes it with NG / 2 8-byte stores (zeros included).  What a dword holds
// depends only on the first non-zero basis index sigma = span - 3, so the
// per-sigma table of kan_sparse.h sits in LDS (built once per workgroup):
// one v_perm_b32 per dword moves the basis value into place, and the silu
// value is or-ed into dword NG - 1 under the entry's mask.
template <int NG>
struct GenS {
    static constexpr bool SPARSE = true;
    static constexpr bool SWZ = false;
    static constexpr int DEPTH = 2;
    static constexpr int NIN = NG == 8 ? 2 : 4;                 // inputs meeting one k-tile
    static constexpr int PPT = 256 * NIN / NTHR;                // pairs per thread
    static constexpr int NPART = PPT;
    static constexpr int RSTEP = NTHR / NIN;
    static constexpr int EQ = sparse_entry_quads<NG>();         // uint4 per table entry
    static_assert(NG == 4 || NG == 6 || NG == 8, "groups per input");
    const uint16_t* x;
    const uint4* tab;
    int q, row0;
    int64_t xrow[PPT];
    uint32_t xs[2][PPT];
    int is[2];
    __device__ GenS(const GemmArgs& a, int tm, int) {
        x = static_cast<const uint16_t*>(a.x);
        q = threadIdx.x % NIN;
        row0 = threadIdx.x / NIN;
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            xrow[j] = (int64_t)min(tm * 256 + row0 + RSTEP * j, a.N - 1) * a.I;
    }
    __device__ __forceinline__ void init(const GemmArgs& a, uint4* aux) {
        for (int e = threadIdx.x; e < a.K + 5; e += NTHR) {
            uint32_t w[4 * EQ];
            sparse_table_entry<NG>(e, a.K, a.base, w);
#pragma unroll
            for (int k = 0; k < EQ; ++k) aux[EQ * e + k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
        }
        tab = aux;
    }
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs& a, int kt) {
        is[SL] = (16 * kt) / NG + q;
        const int i = min(is[SL], a.I - 1);
#pragma unroll
        for (int j = 0; j < PPT; ++j) xs[SL][j] = raw_bits(x, xrow[j] + i);
    }
    // Pair j: the input's index bytes, then its block.
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* row = S + (row0 + RSTEP * j) * PITCH;
        const int i = is[SL];
        const int gofs = i * NG - 16 * kt;                      // tile group of the input's group 0 (even)
        const float xv = raw_to_float<uint16_t>(xs[SL][j]);
        float u;
        const int sig = span_u(xv, a.g, u) - 3;
        const int e = i >= a.I ? a.K + 4 : ((unsigned)(sig + 3) <= (unsigned)(a.K + 2) ? sig + 3 : a.K + 3);
        uint32_t w[4 * EQ];
#pragma unroll
        for (int k = 0; k < EQ; ++k) {
            const uint4 t = tab[EQ * e + k];
            w[4 * k] = t.x, w[4 * k + 1] = t.y, w[4 * k + 2] = t.z, w[4 * k + 3] = t.w;
        }
        const int nb0 = (gofs + 16) >> 1;
#pragma unroll
        for (int c = 0; c < NG / 2; ++c) row[128 + ((nb0 + c) & 15)] = (char)(w[NG] >> (8 * c));
        float b0, b1, b2, b3;
        pieces_fast(u, b0, b1, b2, b3);
        const uint32_t p01 = Traits<uint16_t>::pk(b0, b1), p23 = Traits<uint16_t>::pk(b2, b3);
        uint32_t d[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) d[g] = __builtin_amdgcn_perm(p23, p01, w[g]);
        d[NG - 1] |= Traits<uint16_t>::pk(0.0f, silu(xv)) & w[NG + 1];
        char* blk = row + 4 * (gofs + 8);
#pragma unroll
        for (int c = 0; c < NG / 2; ++c) *reinterpret_cast<uint2*>(blk + 8 * c) = make_uint2(d[2 * c], d[2 * c + 1]);
        if constexpr (RF && j == NPART - 1) fetch<SL>(a, ktn);
    }
};

// Forward A operand of the 2-D layer in 2:4 structured-sparse form (bf16,
// G = 5: K1 = 8, so a pair's 64 columns are exactly one k-tile).  Column
// (m, n) of a pair is logical k = 8 m + 4 (n & 1) + (n >> 1): group 2 m +
// (n & 1), position n >> 1, so the 4 consecutive n of a span put exactly 2
// values into each of the two groups of row m (the coefficient operand is
// packed in the same order).  A group's two stored values sit at positions
// c, c + 1 with c = clamp(first position, 0, 2), zeros filling a position
// that holds none (n outside [0, 8) at the grid's edge).  Two lanes build a
// row: lane half h the 8 groups of m-rows 4 h .. 4 h + 3, stored with the
// row's values at bytes 32 + 32 h (GenS's layout for a k-tile-aligned
// input) and their nibbles at bytes 136 + 4 h.
struct GenS2 {
    static constexpr bool SPARSE = true;
    static constexpr int DEPTH = 2;
    static constexpr int NPART = 1;
    const uint16_t* x;
    int h, row;
    int64_t xrow;
    uint32_t x1s[2], x2s[2];
    __device__ GenS2(const GemmArgs& a, int tm, int) {
        x = static_cast<const uint16_t*>(a.x);
        h = threadIdx.x & 1;
        row = threadIdx.x >> 1;
        xrow = (int64_t)min(tm * 256 + row, a.N - 1) * a.xI;
    }
    __device__ __forceinline__ void init(const GemmArgs&, uint4*) {}
    template <int SL>
    __device__ __forceinline__ void fetch(const GemmArgs&, int kt) {
        x1s[SL] = raw_bits(x, xrow + 2 * kt);            // pair kt
        x2s[SL] = raw_bits(x, xrow + 2 * kt + 1);
    }
    template <int SL, bool RF, int j>
    __device__ __forceinline__ void part(const GemmArgs& a, char* S, int kt, int ktn) {
        char* r0 = S + row * PITCH;
        float u1, u2;
        const int s1 = min(span_u(raw_to_float<uint16_t>(x1s[SL]), a.g, u1), 11);
        const int s2 = min(span_u(raw_to_float<uint16_t>(x2s[SL]), a.g, u2), 11);
        float w1[4], w2[4];
        pieces_fast(u1, w1[0], w1[1], w1[2], w1[3]);
        pieces_fast(u2, w2[0], w2[1], w2[2], w2[3]);
        const int n0 = s2 - 3;                          // first n of the span
        uint32_t d[8], nib = 0;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            // the group's two n: n0 + ql and n0 + ql + 2, ql = 0 when g has n0's parity
            const int ql = (g == (n0 & 1)) ? 0 : 1;
            const int nl = n0 + ql, pl = nl >> 1;
            const int c = min(max(pl, 0), 2);
            const bool vl = (unsigned)nl < 8u, vh = (unsigned)(nl + 2) < 8u;
            const float wl = ql ? w2[1] : w2[0], wh = ql ? w2[3] : w2[2];
            const float v0 = (vl && pl == c) ? wl : (vh && pl + 1 == c) ? wh : 0.0f;
            const float v1 = (vh && pl + 1 == c + 1) ? wh : (vl && pl == c + 1) ? wl : 0.0f;
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int r = 4 * h + mm - (s1 - 3);       // basis index of m = 4 h + mm
                const float wr = r == 0 ? w1[0] : r == 1 ? w1[1] : r == 2 ? w1[2] : r == 3 ? w1[3] : 0.0f;
                d[2 * mm + g] = Traits<uint16_t>::pk(wr * v0, wr * v1);
                nib |= (uint32_t)(c | ((c + 1) << 2)) << (4 * (2 * mm + g));
            }
        }
        *reinterpret_cast<uint4*>(r0 + 32 + 32 * h) = make_uint4(d[0], d[1], d[2], d[3]);
        *reinterpret_cast<uint4*>(r0 + 48 + 32 * h) = make_uint4(d[4], d[5], d[6], d[7]);
        *reinterpret_cast<uint32_t*>(r0 + 136 + 4 * h) = nib;
        if constexpr (RF) fetch<SL>(a, ktn);
    }
};

typedef f32x16 Acc[2][4];

// ---- epilogues ----
// acc[fi][fj][r] holds D[wm + 32 fi + 8 (r / 4) + 4 (lane / 32) + r % 4][wn + 32 fj + lane % 32]
// with wm = 64 (wave / 2), wn = 128 (wave % 2).
__device__ __forceinline__ int acc_row(int fi, int r) { return 32 * fi + 8 * (r >> 2) + (r & 3); }

struct EpiY {
    template <typename TS>
    __device__ static void run(const GemmArgs& a, Acc& acc, int tm, int tn, char*) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int r0 = tm * 256 + (wave >> 1) * 64 + 4 * (lane >> 5);
        const int c0 = tn * 256 + (wave & 1) * 128 + (lane & 31);
#pragma unroll
        for (int fi = 0; fi < 2; ++fi)
#pragma unroll
            for (int fj = 0; fj < 4; ++fj) {
                const int col = c0 + 32 * fj;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = r0 + acc_row(fi, r);
                    if (row < a.N && col < a.O) a.out0[(int64_t)row * a.O + col] = acc[fi][fj][r];
                }
            }
    }
};

struct EpiDC {
    template <typename TS>
    __device__ static void run(const GemmArgs& a, Acc& acc, int tm, int tn, char*) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int r0 = tm * 256 + (wave >> 1) * 64 + 4 * (lane >> 5);
        const int c0 = tn * 256 + (wave & 1) * 128 + (lane & 31);
#pragma unroll
        for (int fj = 0; fj < 4; ++fj) {
            const int n = c0 + 32 * fj;
            if (n >= a.IKb) continue;
            const int i = n / a.Kb, m = n - i * a.Kb;
            const bool spline = m < a.K;
            if (spline ? !a.out0 : !a.out1) continue;
#pragma unroll
            for (int fi = 0; fi < 2; ++fi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = r0 + acc_row(fi, r);
                    if (j >= a.O) continue;
                    if (spline) a.out0[((int64_t)j * a.I + i) * a.K + m] = acc[fi][fj][r];
                    else a.out1[(int64_t)j * a.I + i] = acc[fi][fj][r];
                }
        }
    }
};

// dx: the P tile is staged through LDS in two phases of 128 rows.  In phase h
// every wave writes its accumulator block fi = h (32 of its 64 rows): LDS row
// (wave / 2) * 32 + rr is tile row (wave / 2) * 64 + 32 h + rr.  Then each
// (row, input) pair of those rows contracts its <= 4 spline columns with B'
// and its silu column with silu'.
struct EpiDX {
    // Tile tn holds P columns 256 tn .. +255 of the inputs i_lo .. i_hi.  An
    // input inside the tile gets its dx written here; one cut by a tile edge
    // gets the partial sum over its columns in this tile written to
    // part[b][tn][0] (the input's tail, cut by the left edge) or [1] (its
    // head), and dx_fixup adds the two.
    template <typename TS>
    __device__ static void run(const GemmArgs& a, Acc& acc, int tm, int tn, char* lds) {
        float* P = reinterpret_cast<float*>(lds);
        const TS* x = static_cast<const TS*>(a.x);
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        const int c0 = tn * 256;
        const int i_lo = c0 / a.Kb;
        const int nin = min((c0 + 255) / a.Kb, a.I - 1) - i_lo + 1;
        const int cw = (wave & 1) * 128 + (lane & 31);
        const int rw = (wave >> 1) * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int fj = 0; fj < 4; ++fj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    P[(rw + acc_row(0, r)) * DX_PITCH + cw + 32 * fj] = acc[h][fj][r];
            __syncthreads();
            // 4 items per pass: their x loads go out together (addresses
            // clamped in bounds, values of items past the end unused)
            const int total = 128 * nin;
            const float inv = 1.0f / (float)nin;   // (e + 0.5) / nin stays 1 / (2 nin) off an integer
#pragma unroll 1
            for (int e0 = t; e0 < total; e0 += 4 * NTHR) {
                float xq[4];
                int rlq[4], ilq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = min(e0 + q * NTHR, total - 1);
                    const int rl = (int)(((float)e + 0.5f) * inv), il = e - rl * nin;
                    const int b = min(tm * 256 + (rl >> 5) * 64 + 32 * h + (rl & 31), a.N - 1);
                    rlq[q] = rl;
                    ilq[q] = il;
                    xq[q] = load_f(x, (int64_t)b * a.I + i_lo + il);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rl = rlq[q], il = ilq[q];
                    const int b = tm * 256 + (rl >> 5) * 64 + 32 * h + (rl & 31);
                    const int i = i_lo + il;
                    const int cb = i * a.Kb - c0;            // tile column of (i, m = 0)
                    if (e0 + q * NTHR < total && b < a.N) {
                        const float xv = xq[q];
                        float u;
                        const int s = span_u(xv, a.g, u);
                        float d[4];
                        dpieces(u, a.g.scale, d[0], d[1], d[2], d[3]);
                        const float* prow = P + rl * DX_PITCH;
                        const int cs = cb + a.K;
                        float v = (a.base && cs >= 0 && cs < 256) ? prow[cs] * silu_prime(xv) : 0.0f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = s - 3 + r, c = cb + m;
                            if (m >= 0 && m < a.K && c >= 0 && c < 256) v = __builtin_fmaf(prow[c], d[r], v);
                        }
                        if (cb >= 0 && cb + a.Kb <= 256) a.out0[(int64_t)b * a.I + i] = v;
                        else a.out1[((int64_t)b * a.tiles_n + tn) * 2 + (cb < 0 ? 0 : 1)] = v;
                    }
                }
            }
            __syncthreads();
        }
    }
};

// dx of the inputs cut by a tile edge: input i = 256 (t + 1) / Kb spans
// tiles t and t + 1 when 256 (t + 1) is not a multiple of Kb; its dx is the
// head partial of tile t plus the tail partial of tile t + 1 (a fixed order).
__global__ void dx_fixup_kernel(const float* __restrict__ part, float* __restrict__ dx, int64_t N, int I,
                                int Kb, int tiles) {
    // one (row b, edge t) per thread, edges fastest: the partials of a row
    // are read in order
    const int edges = tiles - 1;
    const int64_t total = N * edges;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = k / edges;
        const int t = (int)(k - b * edges);
        const int64_t c = 256 * (int64_t)(t + 1);
        if (c % Kb == 0 || c / Kb >= I) continue;
        dx[b * I + c / Kb] = part[(b * tiles + t) * 2 + 1] + part[(b * tiles + t + 1) * 2];
    }
}

// dx of the 2-D layer: EpiDX with pairs.  Each (row, pair) of the staged P
// rows contracts its <= 16 columns with B'(x1) B(x2) for dx[b, 2p] and with
// B(x1) B'(x2) for dx[b, 2p+1]: with a_r = sum_q P[m_r, n_q] b_q(u2) and
// d_r = sum_q P[m_r, n_q] b'_q(u2), dx[b, 2p] = sum_r b'_r(u1) a_r and
// dx[b, 2p+1] = sum_r b_r(u1) d_r.  A pair cut by a tile edge writes both
// partial sums to part[b][tn][side][0..1].
struct EpiDX2 {
    template <typename TS>
    __device__ static void run(const GemmArgs& a, Acc& acc, int tm, int tn, char* lds) {
        float* P = reinterpret_cast<float*>(lds);
        const TS* x = static_cast<const TS*>(a.x);
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        const int K1 = a.g.G + 3;
        const int c0 = tn * 256;
        const int p_lo = c0 / a.Kb;
        const int np = min((c0 + 255) / a.Kb, a.I - 1) - p_lo + 1;
        const int cw = (wave & 1) * 128 + (lane & 31);
        const int rw = (wave >> 1) * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int fj = 0; fj < 4; ++fj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    P[(rw + acc_row(0, r)) * DX_PITCH + cw + 32 * fj] = acc[h][fj][r];
            __syncthreads();
#pragma unroll 1
            for (int e = t; e < 128 * np; e += NTHR) {
                const int rl = e / np, pl = e - rl * np;
                const int b = tm * 256 + (rl >> 5) * 64 + 32 * h + (rl & 31);
                const int p = p_lo + pl;
                const int cb = p * a.Kb - c0;            // tile column of (p, 0, 0)
                if (b < a.N) {
                    const int64_t xo = (int64_t)b * a.xI + 2 * p;
                    const float x1 = load_f(x, xo), x2 = load_f(x, xo + 1);
                    float u1, u2;
                    const int s1 = min(span_u(x1, a.g, u1), K1 + 3), s2 = min(span_u(x2, a.g, u2), K1 + 3);
                    float w1[4], d1[4], w2[4], d2[4];
                    pieces(u1, w1[0], w1[1], w1[2], w1[3]);
                    pieces(u2, w2[0], w2[1], w2[2], w2[3]);
                    dpieces(u1, a.g.scale, d1[0], d1[1], d1[2], d1[3]);
                    dpieces(u2, a.g.scale, d2[0], d2[1], d2[2], d2[3]);
                    const float* prow = P + rl * DX_PITCH;
                    float v1 = 0.0f, v2 = 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = s1 - 3 + r;
                        float ar = 0.0f, dr = 0.0f;
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            const int n = s2 - 3 + qq, c = cb + m * K1 + n;
                            if ((unsigned)m < (unsigned)K1 && (unsigned)n < (unsigned)K1 && (unsigned)c < 256u) {
                                ar = __builtin_fmaf(prow[c], w2[qq], ar);
                                dr = __builtin_fmaf(prow[c], d2[qq], dr);
                            }
                        }
                        v1 = __builtin_fmaf(d1[r], ar, v1);
                        v2 = __builtin_fmaf(w1[r], dr, v2);
                    }
                    if (cb >= 0 && cb + a.Kb <= 256) {
                        a.out0[xo] = v1;
                        a.out0[xo + 1] = v2;
                    } else {
                        float* pp = a.out1 + (((int64_t)b * a.tiles_n + tn) * 2 + (cb < 0 ? 0 : 1)) * 2;
                        pp[0] = v1;
                        pp[1] = v2;
                    }
                }
            }
            __syncthreads();
        }
    }
};

// dx of a degree-D layer: EpiDX with the D + 1 derivatives of local_basis_rt.
struct EpiDXK {
    template <typename TS>
    __device__ static void run(const GemmArgs& a, Acc& acc, int tm, int tn, char* lds) {
        float* P = reinterpret_cast<float*>(lds);
        const TS* x = static_cast<const TS*>(a.x);
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        const int D = a.deg;
        const int c0 = tn * 256;
        const int i_lo = c0 / a.Kb;
        const int nin = min((c0 + 255) / a.Kb, a.I - 1) - i_lo + 1;
        const int cw = (wave & 1) * 128 + (lane & 31);
        const int rw = (wave >> 1) * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int fj = 0; fj < 4; ++fj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    P[(rw + acc_row(0, r)) * DX_PITCH + cw + 32 * fj] = acc[h][fj][r];
            __syncthreads();
#pragma unroll 1
            for (int e = t; e < 128 * nin; e += NTHR) {
                const int rl = e / nin, il = e - rl * nin;
                const int b = tm * 256 + (rl >> 5) * 64 + 32 * h + (rl & 31);
                const int i = i_lo + il;
                const int cb = i * a.Kb - c0;
                if (b < a.N) {
                    const float xv = load_f(x, (int64_t)b * a.I + i);
                    float u;
                    const int s = min(span_u(xv, a.g, u), a.K + D);
                    float bb[6], d[6];
                    local_basis_rt(u, a.g.scale, D, bb, d);
                    const float* prow = P + rl * DX_PITCH;
                    const int cs = cb + a.K;
                    float v = (a.base && cs >= 0 && cs < 256) ? prow[cs] * silu_prime(xv) : 0.0f;
#pragma unroll
                    for (int r = 0; r < 6; ++r) {
                        const int m = s - D + r, c = cb + m;
                        if (r <= D && m >= 0 && m < a.K && c >= 0 && c < 256) v = __builtin_fmaf(prow[c], d[r], v);
                    }
                    if (cb >= 0 && cb + a.Kb <= 256) a.out0[(int64_t)b * a.I + i] = v;
                    else a.out1[((int64_t)b * a.tiles_n + tn) * 2 + (cb < 0 ? 0 : 1)] = v;
                }
            }
            __syncthreads();
        }
    }
};

// dx of the pairs cut by a tile edge (the 2-D layer): pair p = 256 (t + 1) /
// Kb spans tiles t and t + 1; each of its two inputs gets the head partial
// of tile t plus the tail partial of tile t + 1.
__global__ void dx_fixup2_kernel(const float* __restrict__ part, float* __restrict__ dx, int64_t N, int P,
                                 int Kb, int tiles) {
    const int edges = tiles - 1;
    const int64_t total = N * edges;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = k / edges;
        const int t = (int)(k - b * edges);
        const int64_t c = 256 * (int64_t)(t + 1);
        if (c % Kb == 0 || c / Kb >= P) continue;
        const int64_t o = b * 2 * P + 2 * (c / Kb);
        const float* head = part + ((b * tiles + t) * 2 + 1) * 2;
        const float* tail = part + ((b * tiles + t + 1) * 2 + 0) * 2;
        dx[o] = head[0] + tail[0];
        dx[o + 1] = head[1] + tail[1];
    }
}

// ---- the contraction kernel ----
template <typename TS, class AOp, class BOp, class Epi>
__global__ __launch_bounds__(NTHR, 1) void gemm_kernel(GemmArgs args) {
    extern __shared__ uint4 lds4[];
    char* lds = reinterpret_cast<char*>(lds4);
    int tm, tn;
    const int slice = tile_coords(args, tm, tn);
    // this workgroup's slice of the k range: the whole range, or one slice
    // of a tail tile, whose output goes to the partial arrays
    int kb = 0, ke = args.nkt;
    if (tm >= args.tiles_m - args.tail) {
        kb = slice * args.nks;
        ke = min(args.nkt, kb + args.nks);
        args.out0 = args.part0 ? args.part0 + (slice * args.ostride0 - args.oshift0) : nullptr;
        args.out1 = args.part1 ? args.part1 + (slice * args.ostride1 - args.oshift1) : nullptr;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
    AOp A(args, tm, tn);
    BOp B(args, tm, tn);
    __shared__ uint4 lds_aux[128];       // per-workgroup table of the sparse generator
    A.init(args, lds_aux);
    B.init(args, lds_aux);
    if (AOp::SPARSE) __syncthreads();
    Acc acc;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fi][fj][r] = 0.0f;

    const int arow = (wm + (lane & 31)) * PITCH + (lane >> 5) * 16;
    const int brow = (wn + (lane & 31)) * PITCH + (lane >> 5) * 16;
    // MFMAs over one staged k-tile: 4 k-steps of 32 bytes per row; after(ks)
    // issues the work placed behind k-step ks.  It runs between the fragment
    // reads and the MFMAs of k-step ks + 1, where it covers the latency of
    // those reads (the last one runs at the end of the tile).
    auto compute = [&](const char* As, const char* Bs, auto&& after) {
      if constexpr (AOp::SPARSE) {
        // 2 sparse steps of 32 logical k; sub-step ks runs step ks / 2 for B
        // blocks 2 (ks % 2), +1.  Lane half h holds logical k 16 h .. +15 of a
        // step in A (8 stored values + 4 index nibbles) and, in B, k 8 h .. +7
        // and 16 + 8 h .. +7 of its column.
        const int h = lane >> 5;
        uint4 sa[2];
        uint2 sidx[2];
#pragma unroll
        for (int f = 0; f < 2; ++f)
            sidx[f] = *reinterpret_cast<const uint2*>(As + arow - h * 16 + f * 32 * PITCH + 136);
        static_for<0, 4>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value, t = ks >> 1, hb = ks & 1;
            if constexpr (hb == 0) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    sa[f] = *reinterpret_cast<const uint4*>(As + arow + f * 32 * PITCH + 32 + 32 * t);
            }
            uint4 fb[2][2];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    fb[f][e] = *reinterpret_cast<const uint4*>(Bs + brow + (2 * hb + f) * 32 * PITCH +
                                                               64 * t + 32 * e);
            if constexpr (ks > 0) after(std::integral_constant<int, ks - 1>());
#pragma unroll
            for (int fi = 0; fi < 2; ++fi) {
                const uint32_t w = t == 0 ? sidx[fi].x : sidx[fi].y;
                const int idx = (int)((w >> (16 * h)) & 0xFFFFu);
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const bf16x16 bv = __builtin_bit_cast(bf16x16, make_u32x8(fb[f][0], fb[f][1]));
                    acc[fi][2 * hb + f] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                        __builtin_bit_cast(bf16x8, sa[fi]), bv, acc[fi][2 * hb + f], idx, 0, 0);
                }
            }
            if constexpr (ks == 3) {
                __builtin_amdgcn_sched_barrier(0);
                after(ksc);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
      } else {
        static_for<0, 4>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            uint4 fa[2], fb[4];
#pragma unroll
            for (int f = 0; f < 4; ++f)
                fb[f] = *reinterpret_cast<const uint4*>(Bs + brow + f * 32 * PITCH + ks * 32);
#pragma unroll
            for (int f = 0; f < 2; ++f)
                fa[f] = *reinterpret_cast<const uint4*>(As + arow + f * 32 * PITCH + ks * 32);
            if constexpr (ks > 0) after(std::integral_constant<int, ks - 1>());
#pragma unroll
            for (int fi = 0; fi < 2; ++fi)
#pragma unroll
                for (int fj = 0; fj < 4; ++fj) Traits<TS>::mma(acc[fi][fj], fa[fi], fb[fj]);
            if constexpr (ks == 3) {
                __builtin_amdgcn_sched_barrier(0);
                after(ksc);
            }
            // pins the k-step's work in place (left free, the scheduler hoists
            // every fragment read of the tile and sinks the stores)
            __builtin_amdgcn_sched_barrier(0);
        });
      }
    };
    // Store k-tile kts from slot SL into stage S, part by part behind the
    // k-steps of the tile being multiplied, and (if RF) refill each operand's
    // slot with tile kts + DEPTH (clamped to the slice's last tile, so every
    // load is in bounds; the extra loads at the end are never stored).
    auto stage = [&](auto slot, auto refill, char* S, int kts, auto ksc) {
        constexpr int SL = decltype(slot)::value;
        constexpr bool RF = decltype(refill)::value;
        constexpr int ks = decltype(ksc)::value;
        const int kna = min(kts + AOp::DEPTH, ke - 1), knb = min(kts + BOp::DEPTH, ke - 1);
        static_for<0, AOp::NPART>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            if constexpr (p * 4 / AOp::NPART == ks) A.template part<SL, RF, p>(args, S, kts, kna);
        });
        static_for<0, BOp::NPART>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            if constexpr (p * 4 / BOp::NPART == ks)
                B.template part<SL, RF, p>(args, S + TILE_BYTES, kts, knb);
        });
    };
    const std::integral_constant<int, 0> slot0;
    const std::integral_constant<int, 1> slot1;
    const std::true_type refill;
    const std::false_type last;
    auto nothing = [](auto) {};
    // Two LDS stages S0, S1.  Invariant at the top of each pass of the loop
    // (kt - kb even): S0 holds tile kt; an operand of DEPTH 2 has slot 1
    // loading tile kt+1 and slot 0 tile kt+2, one of DEPTH 1 has its slot
    // loading tile kt+1.  While tile kt is multiplied from S0, tile kt+1 goes
    // into S1 and the slots refill; then the same with the stages swapped.
    char* S0 = lds;
    char* S1 = lds + STAGE_BYTES;
    A.template fetch<0>(args, kb);
    B.template fetch<0>(args, kb);
    if (AOp::DEPTH == 2) A.template fetch<1>(args, min(kb + 1, ke - 1));
    if (BOp::DEPTH == 2) B.template fetch<1>(args, min(kb + 1, ke - 1));
    static_for<0, 4>([&](auto ksc) { stage(slot0, refill, S0, kb, ksc); });
    __syncthreads();
    int kt = kb;
    for (; kt + 2 < ke; kt += 2) {
        compute(S0, S0 + TILE_BYTES, [&](auto ks) { stage(slot1, refill, S1, kt + 1, ks); });
        __syncthreads();
        compute(S1, S1 + TILE_BYTES, [&](auto ks) { stage(slot0, refill, S0, kt + 2, ks); });
        __syncthreads();
    }
    // Last one or two tiles.  Tile kt+1 may not exist: its store then only
    // writes the free stage S1 (every load behind it is clamped in bounds).
    compute(S0, S0 + TILE_BYTES, [&](auto ks) { stage(slot1, last, S1, kt + 1, ks); });
    __syncthreads();
    if (kt + 1 < ke) compute(S1, S1 + TILE_BYTES, nothing);
    __syncthreads();
    Epi::template run<TS>(args, acc, tm, tn, lds);
}

// 4 consecutive stored elements at p (8 bytes of bf16, 16 of float; p aligned to that)
__device__ __forceinline__ void store4(uint16_t* p, const uint16_t (&o)[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                              (uint32_t)o[2] | ((uint32_t)o[3] << 16));
}
__device__ __forceinline__ void store4(float* p, const float (&o)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

// ---- packing ----
// The loaded operands are stored blocked: element (row r, k) of an operand
// with nk = K / BK k-tiles sits at ((r / 256) * nk + k / BK) * 256 * BK +
// (r % 256) * BK + k % BK (elements), so each k-tile of each 256-row tile is
// one contiguous block.
template <typename TS>
__device__ __forceinline__ int64_t blk(int64_t r, int64_t k, int64_t nk) {
    constexpr int BK = Traits<TS>::BK;
    return ((r >> 8) * nk + k / BK) * (256 * BK) + (r & 255) * BK + k % BK;
}

// C'[j][k], k = i * Kb + m: C[j, i, m] for m < K, W_base[j, i] for m = K; zero
// outside [0, O) x [0, I*Kb).  Rows j < Opad, k < nk * BK.  One block row
// per j, 4 consecutive k per thread.
template <typename TS>
__global__ void pack_fwd_kernel(const TS* __restrict__ C, const TS* __restrict__ W,
                                TS* __restrict__ cp, int O, int I, int K, int Kb, int64_t nk,
                                int64_t Opad) {
    const int64_t IKb = (int64_t)I * Kb;
    const int64_t Kf = nk * Traits<TS>::BK;
    for (int64_t j = blockIdx.y; j < Opad; j += gridDim.y) {
        // 4 consecutive k of one k-tile (Kf and BK are multiples of 4): one store
        for (int64_t k0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; k0 < Kf;
             k0 += (int64_t)gridDim.x * blockDim.x * 4) {
            int i = (int)(k0 / Kb), m = (int)(k0 - (int64_t)i * Kb);
            TS v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t k = k0 + e;
                v[e] = TS(0);
                if (j < O && k < IKb)
                    v[e] = m < K ? C[((int64_t)j * I + i) * K + m] : W[(int64_t)j * I + i];
                if (++m == Kb) { m = 0; ++i; }
            }
            store4(cp + blk<TS>(j, k0, nk), v);
        }
    }
}

// C' for the sparse forward (bf16): input i owns the Kb8 = 4 NG columns
// i Kb8 + 4 g + p, holding its basis column c = p NG + g - dl (C for
// 0 <= c < K, W_base for c = K when there is a base branch, zero otherwise;
// dl = sparse_group_shift); zero outside [0, O) x [0, I Kb8).  Rows j < Opad,
// k < nk * 64.
__global__ void pack_fwd_sparse_kernel(const uint16_t* __restrict__ C, const uint16_t* __restrict__ W,
                                       uint16_t* __restrict__ cp, int O, int I, int K, int base,
                                       int NG, int dl, int64_t nk, int64_t Opad) {
    // one group (4 consecutive k: columns g - dl, NG + g - dl, ... of one
    // input) per thread, stored as one 8-byte word
    const int Kb8 = 4 * NG;
    const int ngroups = (int)(nk * 16);
    for (int64_t j = blockIdx.y; j < Opad; j += gridDim.y) {
        for (int gg = blockIdx.x * blockDim.x + threadIdx.x; gg < ngroups; gg += gridDim.x * blockDim.x) {
            const int k0 = 4 * gg;
            const int i = k0 / Kb8;
            const int g = (k0 - i * Kb8) >> 2;
            uint16_t v[4] = {0, 0, 0, 0};
            if (j < O && i < I) {
                const uint16_t* crow = C + ((int64_t)j * I + i) * K;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int c = p * NG + g - dl;
                    if (c < 0) continue;
                    if (c < K) v[p] = crow[c];
                    else if (c == K && base) v[p] = W[(int64_t)j * I + i];
                }
            }
            *reinterpret_cast<uint2*>(cp + blk<uint16_t>(j, k0, nk)) =
                make_uint2(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16));
        }
    }
}

// C' of the 2-D layer for its sparse forward (bf16, K1 = 8): pair p owns the
// 64 logical columns p 64 + 8 m + 4 (n & 1) + (n >> 1) (GenS2's order); zero
// outside [0, O) x [0, P).  Rows j < Opad, k < nk * 64.
__global__ void pack_fwd_pair_sparse_kernel(const uint16_t* __restrict__ C, uint16_t* __restrict__ cp, int O,
                                            int P, int64_t nk, int64_t Opad) {
    const int64_t Kf = nk * 64;
    for (int64_t j = blockIdx.y; j < Opad; j += gridDim.y) {
        for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < Kf;
             k += (int64_t)gridDim.x * blockDim.x) {
            const int p = (int)(k >> 6), l = (int)(k & 63);
            const int m = l >> 3, n = 2 * (l & 3) + ((l >> 2) & 1);
            uint16_t v = 0;
            if (j < O && p < P) v = C[(((int64_t)j * P + p) * 8 + m) * 8 + n];
            cp[blk<uint16_t>(j, k, nk)] = v;
        }
    }
}

// dx B operand: row R < tiles_dx * 256 is column R of C' (zero for R >= I Kb);
// k runs over j < nk * BK.  64 rows x 64 j per block through an LDS tile,
// written back 16 bytes (consecutive j of one row) per thread.  I Kb is
// below the planner's index limit, so column indices fit in 32 bits.
template <typename TS>
__global__ void pack_bwd_kernel(const TS* __restrict__ C, const TS* __restrict__ W,
                                TS* __restrict__ cpt, int O, int I, int K, int Kb, int64_t nk) {
    constexpr int V = 16 / (int)sizeof(TS);               // elements per 16-byte store
    __shared__ TS tile[64][66];
    const uint32_t R0 = blockIdx.x * 64u;
    const int j0 = blockIdx.y * 64;
    const uint32_t IKb = (uint32_t)I * (uint32_t)Kb;
    const int t = threadIdx.x;
    for (int e = t; e < 64 * 64; e += 256) {
        const int jj = e >> 6, kk = e & 63;
        const int j = j0 + jj;
        const uint32_t k = R0 + kk;
        TS v = TS(0);
        if (j < O && k < IKb) {
            const uint32_t i = k / (uint32_t)Kb, m = k - i * (uint32_t)Kb;
            v = (int)m < K ? C[((int64_t)j * I + i) * K + m] : W[(int64_t)j * I + i];
        }
        tile[jj][kk] = v;
    }
    __syncthreads();
    for (int e = t; e < 64 * 64 / V; e += 256) {
        const int kk = e / (64 / V), jq = (e % (64 / V)) * V;
        union { TS v[V]; uint4 q; } w;
#pragma unroll
        for (int q = 0; q < V; ++q) w.v[q] = tile[jq + q][kk];
        *reinterpret_cast<uint4*>(cpt + blk<TS>(R0 + kk, j0 + jq, nk)) = w.q;
    }
}

template <typename TS> __device__ __forceinline__ TS to_store(float v);
template <> __device__ __forceinline__ float to_store<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_store<uint16_t>(float v) { return f2bf(v); }

// dy (float32 [N, O]) -> dx A operand dyp (rows b < Npad, k = j < Opad) and dC
// A operand dyT (rows j < Opad, k = b < Npad) in the storage dtype,
// zero-padded; 64 x 64 tiles through LDS.
template <typename TS>
__global__ void prep_dy_kernel(const float* __restrict__ dy, TS* __restrict__ dyp,
                               TS* __restrict__ dyt, int N, int O, int64_t Npad, int64_t Opad) {
    __shared__ TS tile[64][68];
    constexpr int BK = Traits<TS>::BK;
    const int64_t b0 = (int64_t)blockIdx.x * 64;
    const int64_t j0 = (int64_t)blockIdx.y * 64;
    const int t = threadIdx.x;
    // 4 consecutive values per lane: one 16-byte load of dy when the row
    // holds them at a 16-byte boundary, and 4 consecutive packed elements
    // (one k-tile holds them: BK and the offsets are multiples of 4)
    const bool vec = (O & 3) == 0;
    for (int e = t; e < 64 * 16; e += 256) {
        const int bb = e >> 4, jq = (e & 15) * 4;
        const int64_t b = b0 + bb, j = j0 + jq;
        float v[4];
        if (vec && b < N && j + 3 < O) {
            const float4 f = *reinterpret_cast<const float4*>(dy + b * O + j);
            v[0] = f.x, v[1] = f.y, v[2] = f.z, v[3] = f.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = (b < N && j + q < O) ? dy[b * O + j + q] : 0.0f;
        }
        TS o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[q] = to_store<TS>(v[q]);
            tile[bb][jq + q] = o[q];
        }
        store4(dyp + blk<TS>(b, j, Opad / BK), o);
    }
    __syncthreads();
    for (int e = t; e < 64 * 16; e += 256) {
        const int jj = e >> 4, bq = (e & 15) * 4;
        TS o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = tile[bq + q][jj];
        store4(dyt + blk<TS>(j0 + jj, b0 + bq, Npad / BK), o);
    }
}

template <typename TS, class AOp, class BOp, class Epi>
hipError_t run_gemm(const GemmArgs& a, hipStream_t s) {
    auto kern = gemm_kernel<TS, AOp, BOp, Epi>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    const int64_t slices = a.tail > 0 ? (a.nkt + a.nks - 1) / a.nks : 0;
    const int64_t blocks = (int64_t)(a.tiles_m - a.tail) * a.tiles_n + (int64_t)a.tail * a.tiles_n * slices;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NTHR), LDS_BYTES, s, a);
    return hipGetLastError();
}

// The operand a generator would build in LDS, built once and written to
// HBM in the blocked layout the copied operands read (k-tile kt of 256-row
// tile T: one contiguous block of 256 rows x 128 bytes at T * tstride + kt *
// BLOCK_BYTES).  One workgroup per (k-tile, tile): the generator fills one
// LDS tile exactly as inside the contraction, then the block is copied out,
// so a contraction that loads it computes the same bits as one that
// generates it.  AOP: the generator is an A operand (its tile is a row tile
// tm), else a B operand (its tile is a column tile tn).
template <typename TS, class Gen, bool AOP>
__global__ __launch_bounds__(NTHR, 1) void gen_pack_kernel(GemmArgs args, char* __restrict__ out,
                                                           int64_t tstride) {
    extern __shared__ uint4 lds4[];
    char* S = reinterpret_cast<char*>(lds4);
    const int kt = blockIdx.x, T = blockIdx.y;
    Gen g(args, AOP ? T : 0, AOP ? 0 : T);
    g.template fetch<0>(args, kt);
    static_for<0, Gen::NPART>([&](auto pc) {
        g.template part<0, false, decltype(pc)::value>(args, S, kt, kt);
    });
    __syncthreads();
    char* dst = out + T * tstride + (int64_t)kt * BLOCK_BYTES;
#pragma unroll
    for (int c = threadIdx.x; c < 256 * 8; c += NTHR)     // 16-byte chunk c % 8 of row c / 8
        *reinterpret_cast<uint4*>(dst + c * 16) = *reinterpret_cast<const uint4*>(S + (c >> 3) * PITCH + (c & 7) * 16);
}

template <typename TS, class Gen, bool AOP>
hipError_t run_gen_pack(const GemmArgs& a, int tiles, int nkt, char* out, hipStream_t s) {
    auto kern = gen_pack_kernel<TS, Gen, AOP>;
    hipLaunchKernelGGL(kern, dim3((unsigned)nkt, (unsigned)tiles), dim3(NTHR), TILE_BYTES, s, a, out,
                       (int64_t)nkt * BLOCK_BYTES);
    return hipGetLastError();
}

// out[e] = sum over slices s = 0 .. P-1, in that order, of part[s n + e],
// added in float64 and rounded once
__global__ void sum_slices_kernel(const float* __restrict__ part, float* __restrict__ out, int64_t n,
                                  int P) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        double v = part[e];
        for (int q = 1; q < P; ++q) v += (double)part[q * n + e];
        out[e] = (float)v;
    }
}

// the same sums, 4 consecutive elements per lane (n a multiple of 4 and
// both arrays 16-byte aligned, so every slice is): 16-byte loads and stores
__global__ void sum_slices4_kernel(const float4* __restrict__ part, float4* __restrict__ out, int64_t n4,
                                   int P) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
         e += (int64_t)gridDim.x * blockDim.x) {
        const float4 f = part[e];
        double v0 = f.x, v1 = f.y, v2 = f.z, v3 = f.w;
        for (int q = 1; q < P; ++q) {
            const float4 g = part[q * n4 + e];
            v0 += (double)g.x, v1 += (double)g.y, v2 += (double)g.z, v3 += (double)g.w;
        }
        out[e] = make_float4((float)v0, (float)v1, (float)v2, (float)v3);
    }
}

hipError_t sum_slices(const float* part, float* out, int64_t n, int P, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const bool vec = (n & 3) == 0 && ((reinterpret_cast<uintptr_t>(part) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    if (vec) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(sum_slices4_kernel, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 16384)),
                           dim3(256), 0, s, reinterpret_cast<const float4*>(part), reinterpret_cast<float4*>(out),
                           n4, P);
    } else {
        hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 16384)),
                           dim3(256), 0, s, part, out, n, P);
    }
    return hipGetLastError();
}

GemmArgs base_args(const Plan& p, const void* x) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.g = p.gk;
    a.N = (int)p.N;
    a.I = (int)p.I;
    a.xI = (int)p.xI;
    a.deg = p.degree;
    a.O = (int)p.O;
    a.K = p.K;
    a.Kb = p.Kb;
    a.base = p.base;
    a.IKb = p.IKb;
    a.group_m = 16;
    a.nks = 1 << 30;     // no tail: every tile runs its whole k range
    return a;
}

}  // namespace

hipError_t launch_pack_fwd(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s) {
    const int64_t per_block = 256 * 4;
    const int64_t nk = p.Kf / p.BK;
    dim3 grid((unsigned)std::min<int64_t>((p.Kf + per_block - 1) / per_block, 65535),
              (unsigned)std::min<int64_t>(p.Opad, 65535));
    if (p.dtype == KAN_F32)
        hipLaunchKernelGGL(pack_fwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(C),
                           static_cast<const float*>(W), static_cast<float*>(cp), (int)p.O, (int)p.I,
                           p.K, p.Kb, nk, p.Opad);
    else
        hipLaunchKernelGGL(pack_fwd_kernel<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(C), static_cast<const uint16_t*>(W),
                           static_cast<uint16_t*>(cp), (int)p.O, (int)p.I, p.K, p.Kb, nk, p.Opad);
    return hipGetLastError();
}

hipError_t launch_pack_fwd_sparse(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s) {
    const int64_t nk = p.Kfs / 64;
    if (p.pair) {
        dim3 grid((unsigned)std::min<int64_t>((p.Kfs + 255) / 256, 65535), (unsigned)std::min<int64_t>(p.Opad, 65535));
        hipLaunchKernelGGL(pack_fwd_pair_sparse_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(C),
                           static_cast<uint16_t*>(cp), (int)p.O, (int)p.I, nk, p.Opad);
        return hipGetLastError();
    }
    dim3 grid((unsigned)std::min<int64_t>((p.Kfs / 4 + 255) / 256, 65535),
              (unsigned)std::min<int64_t>(p.Opad, 65535));
    hipLaunchKernelGGL(pack_fwd_sparse_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(C),
                       static_cast<const uint16_t*>(W), static_cast<uint16_t*>(cp), (int)p.O, (int)p.I,
                       p.K, p.base, p.NG, sparse_group_shift(p.NG, p.K, p.base), nk, p.Opad);
    return hipGetLastError();
}

hipError_t launch_pack_bwd(const Plan& p, const void* C, const void* W, void* cpt, hipStream_t s) {
    dim3 grid((unsigned)(p.tiles_dx * 256 / 64), (unsigned)(p.Opad / 64));
    const int64_t nk = p.Opad / p.BK;
    if (p.dtype == KAN_F32)
        hipLaunchKernelGGL(pack_bwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(C),
                           static_cast<const float*>(W), static_cast<float*>(cpt), (int)p.O, (int)p.I,
                           p.K, p.Kb, nk);
    else
        hipLaunchKernelGGL(pack_bwd_kernel<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(C), static_cast<const uint16_t*>(W),
                           static_cast<uint16_t*>(cpt), (int)p.O, (int)p.I, p.K, p.Kb, nk);
    return hipGetLastError();
}

hipError_t launch_prep_dy(const Plan& p, const float* dy, void* dyp, void* dyt, hipStream_t s) {
    dim3 grid((unsigned)(p.Npad / 64), (unsigned)(p.Opad / 64));
    if (p.dtype == KAN_F32)
        hipLaunchKernelGGL(prep_dy_kernel<float>, grid, dim3(256), 0, s, dy, static_cast<float*>(dyp),
                           static_cast<float*>(dyt), (int)p.N, (int)p.O, p.Npad, p.Opad);
    else
        hipLaunchKernelGGL(prep_dy_kernel<uint16_t>, grid, dim3(256), 0, s, dy,
                           static_cast<uint16_t*>(dyp), static_cast<uint16_t*>(dyt), (int)p.N, (int)p.O,
                           p.Npad, p.Opad);
    return hipGetLastError();
}

// Inputs that can meet one k-tile of the forward: ceil((BK - 1) / Kb) + 1.
static int fwd_nin(const Plan& p) { return (p.BK - 1 + p.Kb - 1) / p.Kb + 1; }

// the truncated-power generator (bf16, KAN_FLAG_TP_FORWARD)
static hipError_t fwd_dispatch_tp(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int n = fwd_nin(p);
    if (n <= 2) return run_gemm<uint16_t, GenT<2>, LoadB, EpiY>(a, s);
    if (n <= 4) return run_gemm<uint16_t, GenT<4>, LoadB, EpiY>(a, s);
    if (n <= 8) return run_gemm<uint16_t, GenT<8>, LoadB, EpiY>(a, s);
    if (n <= 16) return run_gemm<uint16_t, GenT<16>, LoadB, EpiY>(a, s);
    return run_gemm<uint16_t, GenT<32>, LoadB, EpiY>(a, s);
}

template <typename TS>
static hipError_t fwd_dispatch(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int n = fwd_nin(p);           // rounded up to a power of two
    if (n <= 2) return run_gemm<TS, GenA<TS, 2>, LoadB, EpiY>(a, s);
    if (n <= 4) return run_gemm<TS, GenA<TS, 4>, LoadB, EpiY>(a, s);
    if (n <= 8) return run_gemm<TS, GenA<TS, 8>, LoadB, EpiY>(a, s);
    if (n <= 16) return run_gemm<TS, GenA<TS, 16>, LoadB, EpiY>(a, s);
    return run_gemm<TS, GenA<TS, 32>, LoadB, EpiY>(a, s);
}

// (inputs per wave NQW, zero-fill instructions per input ZR) of the dC
// generator, from Kb: the 256-row tile meets ceil(255 / Kb) + 1 inputs, dealt
// to 8 waves: Kb 4..8 needs up to 9 inputs per wave, 9..16 up to 4, larger Kb
// up to 2.
static int dc_nqw(const Plan& p) { return ((255 + p.Kb - 1) / p.Kb + 1 + 7) / 8; }

template <typename TS>
static hipError_t dc_dispatch(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int zr = (p.Kb + 7) / 8;
    const int nq = dc_nqw(p);
    if (zr <= 1 && nq <= 10) return run_gemm<TS, LoadA, GenB<TS, 10, 1>, EpiDC>(a, s);
    if (zr <= 2 && nq <= 4) return run_gemm<TS, LoadA, GenB<TS, 4, 2>, EpiDC>(a, s);
    if (zr <= 3 && nq <= 2) return run_gemm<TS, LoadA, GenB<TS, 2, 3>, EpiDC>(a, s);
    if (zr <= 4 && nq <= 2) return run_gemm<TS, LoadA, GenB<TS, 2, 4>, EpiDC>(a, s);
    if (zr <= 7 && nq <= 2) return run_gemm<TS, LoadA, GenB<TS, 2, 7>, EpiDC>(a, s);
    return run_gemm<TS, LoadA, GenB<TS, 2, 32>, EpiDC>(a, s);
}

template <typename TS>
static hipError_t fwd_dispatch_pair(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int n = fwd_nin(p);           // pairs meeting a k-tile, rounded up to a power of two
    if (n <= 2) return run_gemm<TS, GenA2<TS, 2>, LoadB, EpiY>(a, s);
    if (n <= 4) return run_gemm<TS, GenA2<TS, 4>, LoadB, EpiY>(a, s);
    return run_gemm<TS, GenA2<TS, 8>, LoadB, EpiY>(a, s);
}

// (pairs per wave, zero-fill instructions per pair) of the 2-D dC generator:
// Kb = 16 meets up to 17 pairs per tile (3 per wave), Kb 25..49 up to 12 (2
// per wave), Kb >= 64 up to 5 (1 per wave).  N1 pairs per wave give one
// (row, pair) item per lane: 1 with bf16's 64-row k-tiles, 2 with float32's 32.
template <typename TS>
static hipError_t dc_dispatch_pair(const Plan& p, const GemmArgs& a, hipStream_t s) {
    constexpr int N1 = 64 / Traits<TS>::BK;
    const int zr = (p.Kb + 7) / 8;
    const int nq = dc_nqw(p);
    if (zr <= 2 && nq <= 4) return run_gemm<TS, LoadA, GenB2<TS, 4, 2>, EpiDC>(a, s);
    if (zr <= 7 && nq <= 2) return run_gemm<TS, LoadA, GenB2<TS, 2, 7>, EpiDC>(a, s);
    if (zr <= 8 && nq <= N1) return run_gemm<TS, LoadA, GenB2<TS, N1, 8>, EpiDC>(a, s);
    if (zr <= 16 && nq <= N1) return run_gemm<TS, LoadA, GenB2<TS, N1, 16>, EpiDC>(a, s);
    return run_gemm<TS, LoadA, GenB2<TS, N1, 32>, EpiDC>(a, s);
}

template <typename TS>
static hipError_t fwd_dispatch_deg(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int n = fwd_nin(p);
    if (n <= 2) return run_gemm<TS, GenAK<TS, 2>, LoadB, EpiY>(a, s);
    if (n <= 4) return run_gemm<TS, GenAK<TS, 4>, LoadB, EpiY>(a, s);
    if (n <= 8) return run_gemm<TS, GenAK<TS, 8>, LoadB, EpiY>(a, s);
    if (n <= 16) return run_gemm<TS, GenAK<TS, 16>, LoadB, EpiY>(a, s);
    return run_gemm<TS, GenAK<TS, 32>, LoadB, EpiY>(a, s);
}

template <typename TS>
static hipError_t dc_dispatch_deg(const Plan& p, const GemmArgs& a, hipStream_t s) {
    const int zr = (p.Kb + 7) / 8;
    const int nq = dc_nqw(p);
    if (zr <= 1 && nq <= 10) return run_gemm<TS, LoadA, GenBK<TS, 10, 1>, EpiDC>(a, s);
    if (zr <= 2 && nq <= 4) return run_gemm<TS, LoadA, GenBK<TS, 4, 2>, EpiDC>(a, s);
    if (zr <= 4 && nq <= 2) return run_gemm<TS, LoadA, GenBK<TS, 2, 4>, EpiDC>(a, s);
    if (zr <= 7 && nq <= 2) return run_gemm<TS, LoadA, GenBK<TS, 2, 7>, EpiDC>(a, s);
    return run_gemm<TS, LoadA, GenBK<TS, 2, 32>, EpiDC>(a, s);
}

static hipError_t fwd_run(const Plan& p, GemmArgs& a, hipStream_t s) {
    if (p.degree != 3) return p.dtype == KAN_F32 ? fwd_dispatch_deg<float>(p, a, s) : fwd_dispatch_deg<uint16_t>(p, a, s);
    if (p.pair) {
        if (p.sparse) return run_gemm<uint16_t, GenS2, LoadB, EpiY>(a, s);
        return p.dtype == KAN_F32 ? fwd_dispatch_pair<float>(p, a, s) : fwd_dispatch_pair<uint16_t>(p, a, s);
    }
    if (p.sparse) {
        if (p.NG == 4) return run_gemm<uint16_t, GenS<4>, LoadB, EpiY>(a, s);
        if (p.NG == 6) return run_gemm<uint16_t, GenS<6>, LoadB, EpiY>(a, s);
        return run_gemm<uint16_t, GenS<8>, LoadB, EpiY>(a, s);
    }
    if (p.dtype == KAN_F32) return fwd_dispatch<float>(p, a, s);
    if (p.tp) return fwd_dispatch_tp(p, a, s);
    return fwd_dispatch<uint16_t>(p, a, s);
}

// the dense bf16 forward of a cubic layer with its basis operand built once
// in HBM (Plan::mat_fwd): the generator as in fwd_dispatch, into a pack
static hipError_t fwd_mat_run(const Plan& p, GemmArgs& a, void* phi, hipStream_t s) {
    const int n = fwd_nin(p);
    char* out = static_cast<char*>(phi);
    hipError_t e;
    if (n <= 2) e = run_gen_pack<uint16_t, GenA<uint16_t, 2>, true>(a, a.tiles_m, a.nkt, out, s);
    else if (n <= 4) e = run_gen_pack<uint16_t, GenA<uint16_t, 4>, true>(a, a.tiles_m, a.nkt, out, s);
    else if (n <= 8) e = run_gen_pack<uint16_t, GenA<uint16_t, 8>, true>(a, a.tiles_m, a.nkt, out, s);
    else if (n <= 16) e = run_gen_pack<uint16_t, GenA<uint16_t, 16>, true>(a, a.tiles_m, a.nkt, out, s);
    else e = run_gen_pack<uint16_t, GenA<uint16_t, 32>, true>(a, a.tiles_m, a.nkt, out, s);
    if (e != hipSuccess) return e;
    a.a = out;
    a.a_tstride = (int64_t)a.nkt * BLOCK_BYTES;
    return run_gemm<uint16_t, LoadA, LoadB, EpiY>(a, s);
}

hipError_t launch_mfma_fwd(const Plan& p, const void* x, const void* cp, void* phi, float* ypart, float* y,
                           hipStream_t s) {
    GemmArgs a = base_args(p, x);
    a.tiles_m = (int)(p.Npad / 256);
    a.tiles_n = (int)(p.Opad / 256);
    a.b = static_cast<const char*>(cp);
    a.nkt = (int)(p.sparse ? p.Kfs / 64 : p.Kf / p.BK);
    a.b_tstride = (int64_t)a.nkt * BLOCK_BYTES;
    a.out0 = y;
    auto run = [&]() { return p.mat_fwd ? fwd_mat_run(p, a, phi, s) : fwd_run(p, a, s); };
    if (p.split_fwd <= 1) return run();
    // the tail rows in split_fwd slices: partials, then a sum in slice order
    const int64_t r0 = first_fwd_row(p), n = fwd_tail_rows(p) * p.O;
    a.tail = (int)p.tail_fwd;
    a.nks = (int)p.nks_fwd;
    a.part0 = ypart;
    a.ostride0 = n;
    a.oshift0 = r0 * p.O;
    hipError_t e = run();
    return e != hipSuccess ? e : sum_slices(ypart, y + r0 * p.O, n, p.split_fwd, s);
}

hipError_t launch_mfma_dx(const Plan& p, const void* x, const void* dyp, const void* cpt,
                          float* part, float* dx, hipStream_t s) {
    GemmArgs a = base_args(p, x);
    a.tiles_m = (int)(p.Npad / 256);
    a.tiles_n = (int)p.tiles_dx;
    a.a = static_cast<const char*>(dyp);
    a.a_tstride = p.Opad / p.BK * BLOCK_BYTES;
    a.b = static_cast<const char*>(cpt);
    a.b_tstride = p.Opad / p.BK * BLOCK_BYTES;
    a.nkt = (int)(p.Opad / p.BK);
    a.out0 = dx;
    a.out1 = part;
    // both operands are copied and equally large per tile: 8 x 4 tiles per
    // 32 resident workgroups of an XCD share each dy and each C'^T tile
    a.group_m = 8;
    if (p.degree != 3) {
        hipError_t e = p.dtype == KAN_F32 ? run_gemm<float, LoadA, LoadB, EpiDXK>(a, s)
                                          : run_gemm<uint16_t, LoadA, LoadB, EpiDXK>(a, s);
        if (e != hipSuccess || p.tiles_dx < 2) return e;
        hipLaunchKernelGGL(dx_fixup_kernel,
                           dim3((unsigned)std::min<int64_t>((p.N * (p.tiles_dx - 1) + 255) / 256, 16384)),
                           dim3(256), 0, s, part, dx, (int64_t)p.N, (int)p.I, p.Kb, (int)p.tiles_dx);
        return hipGetLastError();
    }
    if (p.pair) {
        hipError_t e = p.dtype == KAN_F32 ? run_gemm<float, LoadA, LoadB, EpiDX2>(a, s)
                                          : run_gemm<uint16_t, LoadA, LoadB, EpiDX2>(a, s);
        if (e != hipSuccess || p.tiles_dx < 2) return e;
        hipLaunchKernelGGL(dx_fixup2_kernel,
                           dim3((unsigned)std::min<int64_t>((p.N * (p.tiles_dx - 1) + 255) / 256, 16384)),
                           dim3(256), 0, s, part, dx, (int64_t)p.N, (int)p.I, p.Kb, (int)p.tiles_dx);
        return hipGetLastError();
    }
    hipError_t e = p.dtype == KAN_F32 ? run_gemm<float, LoadA, LoadB, EpiDX>(a, s)
                                      : run_gemm<uint16_t, LoadA, LoadB, EpiDX>(a, s);
    if (e != hipSuccess || p.tiles_dx < 2) return e;
    hipLaunchKernelGGL(dx_fixup_kernel,
                       dim3((unsigned)std::min<int64_t>((p.N * (p.tiles_dx - 1) + 255) / 256, 16384)),
                       dim3(256), 0, s, part, dx, (int64_t)p.N, (int)p.I, p.Kb, (int)p.tiles_dx);
    return hipGetLastError();
}

// dC of a cubic bf16 layer with its basis operand built once in HBM
// (Plan::mat_dc): the generator as in dc_dispatch (dc_dispatch_pair for the
// 2-D layer), into a pack
static hipError_t dc_mat_run(const Plan& p, GemmArgs& a, void* phit, hipStream_t s) {
    const int zr = (p.Kb + 7) / 8;
    const int nq = dc_nqw(p);
    char* out = static_cast<char*>(phit);
    hipError_t e;
    if (p.pair) {   // the generator dc_dispatch_pair takes for bf16 (one item per lane)
        if (zr <= 2 && nq <= 4) e = run_gen_pack<uint16_t, GenB2<uint16_t, 4, 2>, false>(a, a.tiles_n, a.nkt, out, s);
        else if (zr <= 7 && nq <= 2) e = run_gen_pack<uint16_t, GenB2<uint16_t, 2, 7>, false>(a, a.tiles_n, a.nkt, out, s);
        else if (zr <= 8 && nq <= 1) e = run_gen_pack<uint16_t, GenB2<uint16_t, 1, 8>, false>(a, a.tiles_n, a.nkt, out, s);
        else if (zr <= 16 && nq <= 1) e = run_gen_pack<uint16_t, GenB2<uint16_t, 1, 16>, false>(a, a.tiles_n, a.nkt, out, s);
        else e = run_gen_pack<uint16_t, GenB2<uint16_t, 1, 32>, false>(a, a.tiles_n, a.nkt, out, s);
    } else if (zr <= 1 && nq <= 10) {
        e = run_gen_pack<uint16_t, GenB<uint16_t, 10, 1>, false>(a, a.tiles_n, a.nkt, out, s);
    } else if (zr <= 2 && nq <= 4) {
        e = run_gen_pack<uint16_t, GenB<uint16_t, 4, 2>, false>(a, a.tiles_n, a.nkt, out, s);
    } else {
        return hipErrorInvalidValue;      // the plan builds 1-D operands for Kb <= 12 only
    }
    if (e != hipSuccess) return e;
    a.b = out;
    a.b_tstride = (int64_t)a.nkt * BLOCK_BYTES;
    return run_gemm<uint16_t, LoadA, LoadB, EpiDC>(a, s);
}

hipError_t launch_mfma_dc(const Plan& p, const void* x, const void* dyt, void* phit, float* cpart, float* dC,
                          float* dW, hipStream_t s) {
    GemmArgs a = base_args(p, x);
    a.tiles_m = (int)(p.Opad / 256);
    a.tiles_n = (int)((p.IKb + 255) / 256);
    a.a = static_cast<const char*>(dyt);
    a.a_tstride = p.Npad / p.BK * BLOCK_BYTES;
    a.nkt = (int)(p.Npad / p.BK);
    a.out0 = dC;
    a.out1 = dW;
    a.group_m = 2;
    auto dispatch = [&]() {
        if (p.mat_dc) return dc_mat_run(p, a, phit, s);
        if (p.degree != 3) return p.dtype == KAN_F32 ? dc_dispatch_deg<float>(p, a, s) : dc_dispatch_deg<uint16_t>(p, a, s);
        if (p.pair) return p.dtype == KAN_F32 ? dc_dispatch_pair<float>(p, a, s) : dc_dispatch_pair<uint16_t>(p, a, s);
        return p.dtype == KAN_F32 ? dc_dispatch<float>(p, a, s) : dc_dispatch<uint16_t>(p, a, s);
    };
    if (p.split_dc <= 1) return dispatch();
    // the tail rows j with the batch in split_dc fixed slices: partials,
    // then a sum in slice order
    const int64_t j0 = first_dc_row(p), rows = dc_tail_rows(p);
    const int64_t nc = rows * p.I * p.K, nw = rows * p.I;
    float* wpart = cpart + p.split_dc * nc;
    a.tail = (int)p.tail_dc;
    a.nks = (int)p.nks_dc;
    a.part0 = dC ? cpart : nullptr;
    a.part1 = dW ? wpart : nullptr;
    a.ostride0 = nc;
    a.ostride1 = nw;
    a.oshift0 = j0 * p.I * p.K;
    a.oshift1 = j0 * p.I;
    hipError_t e = dispatch();
    if (e == hipSuccess && dC) e = sum_slices(cpart, dC + j0 * p.I * p.K, nc, p.split_dc, s);
    if (e == hipSuccess && dW) e = sum_slices(wpart, dW + j0 * p.I, nw, p.split_dc, s);
    return e;
}

}  // namespace kan
