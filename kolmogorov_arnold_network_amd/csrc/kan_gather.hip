// Local-basis kernels on the vector ALUs (gfx950), plus the standalone basis
// evaluation, the bf16 cast and a zero fill.
//
// "Local 4-basis lookup instead of dense K-basis computation" (InKAN project
// page, "Why InKAN?"): for each (row b, input i) only the span s and the D + 1
// non-zero pieces of degree D (4 for the cubic layer) are formed; the
// contractions then gather the coefficients C[j, i, s-D .. s].  Arithmetic is
// float32 (the forward adds its partial sums in float64) and every reduction
// runs in a fixed order without atomics.
#include <type_traits>

#include "kan_internal.h"

namespace kan {

namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Standalone basis: dense B[k, m] and dB[k, m], one element per thread (m
// fastest, so the stores are contiguous; n K < 2^31 is checked by the
// caller).  Local form (TP false): the span and the 4 pieces of x[k], element
// m taking piece m - (s - 3) or 0.  Truncated-power form (TP true): every
// element on its own from u = (x[k] - t_m) / h, with no span.
template <typename TS, bool TP>
__global__ void basis_eval_kernel(GridK g, int64_t n, const TS* __restrict__ x,
                                  float* __restrict__ B, float* __restrict__ dB) {
    const int K = g.G + 3;
    const int total = (int)(n * K);
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
        const int k = e / K, m = e - k * K;
        const float xv = load_f(x, k);
        float b, d;
        if constexpr (TP) {
            tp_basis(__builtin_fmaf(xv, g.scale, g.shift - (float)m), g.scale, b, d);
        } else {
            float u;
            const int r = m - (span_u(xv, g, u) - 3);
            float p[4], q[4];
            pieces(u, p[0], p[1], p[2], p[3]);
            dpieces(u, g.scale, q[0], q[1], q[2], q[3]);
            b = r == 0 ? p[0] : r == 1 ? p[1] : r == 2 ? p[2] : r == 3 ? p[3] : 0.0f;
            d = r == 0 ? q[0] : r == 1 ? q[1] : r == 2 ? q[2] : r == 3 ? q[3] : 0.0f;
        }
        if (B) B[e] = b;
        if (dB) dB[e] = d;
    }
}

// ---- basis functions of degree D (the layer kernels' pieces for D != 3) ----
// The D + 1 non-zero uniform B-splines of degree D on a knot span, by local
// coordinate u in [0, 1]: value r belongs to basis function s - D + r.  They
// come from the degree-by-degree recurrence on uniform knots,
//     N^q_r = ((u + q - r) N^{q-1}_{r-1} + (r + 1 - u) N^{q-1}_r) / q,
// whose terms are all non-negative on [0, 1] (no alternating sum), and
// the derivatives from one degree lower: dN^D_r/dx = (N^{D-1}_{r-1} -
// N^{D-1}_r) / h.
template <int D>
__device__ __forceinline__ void local_basis(float u, float scale, float b[D + 1], float d[D + 1]) {
    float N[D + 1];
    N[0] = 1.0f;
#pragma unroll
    for (int q = 1; q <= D; ++q) {
        if (q == D) {
#pragma unroll
            for (int r = 0; r <= D; ++r)
                d[r] = ((r >= 1 ? N[r - 1] : 0.0f) - (r <= D - 1 ? N[r] : 0.0f)) * scale;
        }
        const float inv = 1.0f / (float)q;
        // descending r: N[r - 1] still holds degree q - 1 when N[r] is replaced
#pragma unroll
        for (int r = q; r >= 0; --r) {
            float v = r >= 1 ? (u + (float)(q - r)) * N[r - 1] : 0.0f;
            if (r <= q - 1) v = __builtin_fmaf((float)(r + 1) - u, N[r], v);
            N[r] = v * inv;
        }
    }
#pragma unroll
    for (int r = 0; r <= D; ++r) b[r] = N[r];
}

// Truncated-power form of one degree-D basis function (FlashKAN project page:
// D + 2 shifted (x)_+^D terms, coordinate clamped to [0, D + 1]):
// u = (x - t_m) / h, B = sum_i (-1)^i C(D+1, i) (u - i)_+^D / D!, and
// B' = sum_i (-1)^i C(D+1, i) (u - i)_+^{D-1} / (D-1)! / h, summed in i order
// (the i = D + 1 term vanishes under the clamp).  At D = 1 the derivative's
// terms are steps (w)_+^0 = [w >= 0], the right-hand derivative, as the
// half-open knot spans have it; each step's sign is taken from its own
// single-rounding FMA x/h + (shift - (m + i)), the test span_u uses for the
// span, since u - i from a rounded u can land on the knot from below.
template <int D>
__device__ __forceinline__ void tp_basis_deg(float x, const GridK& g, int m, float& b, float& d) {
    constexpr float fact[6] = {1.0f, 1.0f, 2.0f, 6.0f, 24.0f, 120.0f};
    const float scale = g.scale;
    const float u_raw = __builtin_fmaf(x, scale, g.shift - (float)m);
    const float u = __builtin_fminf(__builtin_fmaxf(u_raw, 0.0f), (float)(D + 1));
    float sb = 0.0f, sd = 0.0f;
    int c = 1;                                   // C(D+1, i)
#pragma unroll
    for (int i = 0; i <= D + 1; ++i) {
        const float sgn = (i & 1) ? -(float)c : (float)c;
        const float w = __builtin_fmaxf(u - (float)i, 0.0f);
        float wp = 1.0f;                         // w^(D-1)
#pragma unroll
        for (int e = 0; e < D - 1; ++e) wp *= w;
        if (i <= D) sb = __builtin_fmaf(sgn, wp * w, sb);
        if (D == 1) sd += __builtin_fmaf(x, scale, g.shift - (float)(m + i)) >= 0.0f ? sgn : 0.0f;
        else if (i <= D) sd = __builtin_fmaf(sgn, wp, sd);
        c = c * (D + 1 - i) / (i + 1);
    }
    b = sb * (1.0f / fact[D]);
    d = sd * (scale / fact[D - 1]);
}

// Dense B, dB [n, G + D] for degree D != 3, one element per thread; g.shift
// places t_0 = lo - D h.
template <typename TS, bool TP, int D>
__global__ void basis_eval_deg_kernel(GridK g, int64_t n, const TS* __restrict__ x,
                                      float* __restrict__ B, float* __restrict__ dB) {
    const int K = g.G + D;
    const int total = (int)(n * K);
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
        const int k = e / K, m = e - k * K;
        const float xv = load_f(x, k);
        float b = 0.0f, d = 0.0f;
        if constexpr (TP) {
            tp_basis_deg<D>(xv, g, m, b, d);
        } else {
            float u;
            const int r = m - (span_u(xv, g, u) - D);
            float bb[D + 1], dd[D + 1];
            local_basis<D>(u, g.scale, bb, dd);
#pragma unroll
            for (int q = 0; q <= D; ++q)
                if (r == q) {
                    b = bb[q];
                    d = dd[q];
                }
        }
        if (B) B[e] = b;
        if (dB) dB[e] = d;
    }
}

// 8 values per lane and step: two 16-byte loads, one 16-byte store (both
// arrays are 16-byte aligned); the last n % 8 values one by one
__global__ void cast_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
    const int64_t n8 = n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n8; k += stride) {
        const float4 a = reinterpret_cast<const float4*>(in)[2 * k];
        const float4 b = reinterpret_cast<const float4*>(in)[2 * k + 1];
        uint4 o;
        o.x = (uint32_t)f2bf(a.x) | ((uint32_t)f2bf(a.y) << 16);
        o.y = (uint32_t)f2bf(a.z) | ((uint32_t)f2bf(a.w) << 16);
        o.z = (uint32_t)f2bf(b.x) | ((uint32_t)f2bf(b.y) << 16);
        o.w = (uint32_t)f2bf(b.z) | ((uint32_t)f2bf(b.w) << 16);
        reinterpret_cast<uint4*>(out)[k] = o;
    }
    for (int64_t k = 8 * n8 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n; k += stride)
        out[k] = f2bf(in[k]);
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x)
        p[k] = 0.0f;
}

// ---------------------------------------------------------------------------
// Layer kernels.  Per (b, i): span-relative coefficient index base and the
// D + 1 weights with the out-of-range ones set to zero, so the inner loops can
// clamp the index and multiply unconditionally.
template <int D>
struct RecD {
    int m0;              // s - D: index of the coefficient that piece 0 multiplies
    float w[D + 1];      // piece r (or its derivative) for m = m0 + r; 0 where m is outside [0, K-1]
    float base;          // silu(x) or silu'(x)
};

template <bool DERIV, int D>
__device__ __forceinline__ RecD<D> make_rec(float xv, const GridK& g) {
    RecD<D> r;
    float u;
    const int s = span_u(xv, g, u);
    float w[D + 1];
    if constexpr (D == 3) {
        if (DERIV) dpieces(u, g.scale, w[0], w[1], w[2], w[3]);
        else pieces(u, w[0], w[1], w[2], w[3]);
    } else {
        float b[D + 1], d[D + 1];
        local_basis<D>(u, g.scale, b, d);
#pragma unroll
        for (int q = 0; q <= D; ++q) w[q] = DERIV ? d[q] : b[q];
    }
    r.m0 = s - D;
    const int K = g.G + D;
#pragma unroll
    for (int q = 0; q <= D; ++q) r.w[q] = (r.m0 + q >= 0 && r.m0 + q < K) ? w[q] : 0.0f;
    r.base = DERIV ? silu_prime(xv) : silu(xv);
    return r;
}

template <int D>
__device__ __forceinline__ RecD<D> zero_rec() {
    RecD<D> r;
    r.m0 = 0;
#pragma unroll
    for (int q = 0; q <= D; ++q) r.w[q] = 0.0f;
    r.base = 0.0f;
    return r;
}

// ---------------------------------------------------------------------------
// Forward.  A block computes R = NT / 4 rows by 64 outputs over one slice of
// the inputs: thread t takes the 4 outputs 4 (t % 16) .. +3 of the rows
// t / 16 + (NT / 16) p, p < 4.  Inputs advance in chunks of IC <= 8 held in
// LDS: the chunk's coefficients for the block's 64 outputs as Cs[ii][m][j]
// (4 outputs of one coefficient row are one 16-byte read), its W_base as
// Ws[ii][j], and one span record per (row, input).  There are two chunk
// buffers: while one chunk is multiplied, the next chunk's coefficients,
// W_base and x are loaded into registers, then written (x as its span record)
// to the other buffer, with one barrier per chunk.
//
// - A thread's sums over a run of at most 8 inputs (one chunk, or several
//   chunks when K is large and a chunk holds fewer than 8 inputs) are
//   float32; each run's sum is added into a float64 accumulator.  In a chain
//   of layers the next layer's B' amplifies forward rounding about tenfold,
//   so the long sum over inputs is kept out of float32.
// - All R rows of the block share one staged chunk, so the coefficient
//   traffic per row, the part of the work that grows with G, falls as R
//   grows.
// - With too few blocks to fill the GPU the inputs are split into slices.
//   Each slice writes float64 partial outputs, which gather_sum_kernel adds
//   in slice order.
constexpr int GF_TJ = kGatherFwdOutputs;

template <int D>
struct alignas(8) RecF {
    int cb;              // LDS index of coefficient row mb of the pair's input, Cs[ii][mb][0]
    float w[D + 1];      // weights of rows mb .. mb + D
    float base;          // silu(x); 0 without the base branch
};

// mb = s - D clamped to [0, K - D - 1], so that rows mb .. mb + D all exist,
// and the pieces shifted by the clamp (zero where a basis index is out of
// range or the span lies off the grid).
template <int D>
__device__ __forceinline__ RecF<D> make_recf(float xv, const GridK& g, int ii, bool base) {
    const RecD<D> r = make_rec<false, D>(xv, g);
    const int K = g.G + D;
    const int mb = clampi(r.m0, 0, K - D - 1);
    RecF<D> f;
    f.cb = (ii * K + mb) * GF_TJ;
#pragma unroll
    for (int q = 0; q <= D; ++q) {
        const int k = mb + q - r.m0;                 // which piece multiplies row mb + q
        float v = 0.0f;
#pragma unroll
        for (int e = 0; e <= D; ++e) v = k == e ? r.w[e] : v;
        f.w[q] = v;
    }
    f.base = base ? r.base : 0.0f;
    return f;
}

template <typename TS, int D, bool BASE, int NT, int MAXQ>
__global__ __launch_bounds__(NT) void gather_fwd_kernel(GatherFwdArgs a) {
    constexpr int R = NT / 4;                        // rows per block
    constexpr int RS = NT / 16;                      // row stride of a thread's 4 rows
    constexpr int NPC = NT / 64;                     // threads sharing one output's coefficient loads
    constexpr int RW = (int)(sizeof(RecF<D>) / 4);
    constexpr int XV = (R * 8 + NT - 1) / NT;        // x loads per thread (IC <= 8)
    constexpr int WV = (GF_TJ * 8 + NT - 1) / NT;    // W_base loads per thread
    constexpr int PG = NT == 1024 ? 1 : 4;           // rows whose LDS reads overlap
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const TS* __restrict__ x = static_cast<const TS*>(a.x);
    const TS* __restrict__ C = static_cast<const TS*>(a.C);
    const TS* __restrict__ W = static_cast<const TS*>(a.W);
    const GridK g = a.g;
    const int K = g.G + D, IC = a.IC, I = a.I, N = a.N, O = a.O;
    const int csz = IC * K * GF_TJ, wsz = BASE ? IC * GF_TJ : 0;
    const int bufsz = csz + wsz + IC * R * RW;       // floats per chunk buffer
    const int t = threadIdx.x;

    // block -> (row block, output block).  Workgroups are dealt to the 8 XCDs
    // in turn; consecutive ids go to one XCD with row blocks fastest, so the
    // blocks an XCD runs together share one output block's coefficients in
    // its L2.
    const int T = a.RB * a.OB;
    const int bid = blockIdx.x, nfull = T / 8, rem = T % 8, xcd = bid % 8;
    const int id = xcd * nfull + min(xcd, rem) + bid / 8;
    const int rb = id % a.RB, ob = id / a.RB;
    const int b0 = rb * R, j0 = ob * GF_TJ;
    const int slice = blockIdx.y;
    const int ib = slice * a.IS, ie = min(I, ib + a.IS);
    const int nch = (ie - ib + IC - 1) / IC;
    const int fold = max(1, 8 / IC);                 // chunks per float32 run

    // Coefficient loads: output jl = t % 64 of the block (an output past O
    // reads output O - 1; its sums are never stored), 4-element pieces
    // k = t / 64 + NPC q of that output's chunk row C[j, i0 .. i0+nic-1, :],
    // each clamped to start inside the row.  Consecutive lanes hold
    // consecutive outputs, so the LDS stores are free of bank conflicts.
    // Loads are issued unconditionally from addresses clamped in bounds where
    // possible (a guarded load into a register that was zeroed first makes
    // the compiler wait for every earlier load); invalid values are zeroed
    // when stored.
    const int jl = t % 64, pc = t / 64;
    const TS* crow = C + (int64_t)min(j0 + jl, O - 1) * I * K;
    float4 cp[MAXQ];
    float xp[XV], wp[WV];
    auto load = [&](int c) {
        const int i0 = ib + c * IC, nic = min(IC, ie - i0);
        const int ick = nic * K;
        const TS* src = crow + (int64_t)i0 * K;
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int k = pc + NPC * q;
            if (4 * k < ick) {
                if (std::is_same<TS, float>::value && ick >= 4) {
                    __builtin_memcpy(&cp[q], reinterpret_cast<const float*>(src) + min(4 * k, ick - 4), 16);
                } else {
                    const int s = ick >= 4 ? min(4 * k, ick - 4) : 0;
                    cp[q].x = load_f(src, min(s + 0, ick - 1));
                    cp[q].y = load_f(src, min(s + 1, ick - 1));
                    cp[q].z = load_f(src, min(s + 2, ick - 1));
                    cp[q].w = load_f(src, min(s + 3, ick - 1));
                }
            }
        }
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int u = t + NT * v, row = u / IC, ii = u - row * IC;
            const bool ok = u < R * IC && b0 + row < N && ii < nic;
            xp[v] = load_f(x, ok ? (int64_t)(b0 + row) * I + i0 + ii : 0);
        }
        if constexpr (BASE) {
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int u = t + NT * v, jj = u / IC, ii = u - jj * IC;
                const bool ok = u < GF_TJ * IC && j0 + jj < O && ii < nic;
                wp[v] = load_f(W, ok ? (int64_t)(j0 + jj) * I + i0 + ii : 0);
            }
        }
    };
    auto store = [&](int c, int buf) {
        float* Cs = smem + buf * bufsz;
        float* Ws = Cs + csz;
        RecF<D>* Rs = reinterpret_cast<RecF<D>*>(Ws + wsz);
        const int i0 = ib + c * IC, nic = min(IC, ie - i0);
        const int ick = nic * K;
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int k = pc + NPC * q;
            if (4 * k < ick) {
                const int s = ick >= 4 ? min(4 * k, ick - 4) : 0;
                const float vv[4] = {cp[q].x, cp[q].y, cp[q].z, cp[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (s + e < ick) Cs[(s + e) * GF_TJ + jl] = vv[e];
            }
        }
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int u = t + NT * v, row = u / IC, ii = u - row * IC;
            if (u < R * IC && ii < nic) {
                RecF<D> r;
                if (b0 + row < N) {
                    r = make_recf<D>(xp[v], g, ii, BASE);
                } else {                             // a row past N: valid index, no weight
                    r.cb = ii * K * GF_TJ;
#pragma unroll
                    for (int q = 0; q <= D; ++q) r.w[q] = 0.0f;
                    r.base = 0.0f;
                }
                Rs[ii * R + row] = r;
            }
        }
        if constexpr (BASE) {
#pragma unroll
            for (int v = 0; v < WV; ++v) {
                const int u = t + NT * v, jj = u / IC, ii = u - jj * IC;
                if (u < GF_TJ * IC && ii < nic) Ws[ii * GF_TJ + jj] = j0 + jj < O ? wp[v] : 0.0f;
            }
        }
    };

    const int jq = t & 15, rq = t >> 4;
    float acc[4][4];
    double accd[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[p][q] = 0.0f;
            accd[p][q] = 0.0;
        }
    load(0);
    store(0, 0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        if (more) load(c + 1);
        const float* Cs = smem + (c & 1) * bufsz;
        const float* Ws = Cs + csz;
        const RecF<D>* Rs = reinterpret_cast<const RecF<D>*>(Ws + wsz);
        const int nic = min(IC, ie - (ib + c * IC));
        for (int ii = 0; ii < nic; ++ii) {
            float4 wv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if constexpr (BASE) wv = *reinterpret_cast<const float4*>(&Ws[ii * GF_TJ + 4 * jq]);
            RecF<D> rr[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) rr[p] = Rs[ii * R + rq + RS * p];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const RecF<D>& r = rr[p];
                const float* cr = Cs + r.cb + 4 * jq;
                // the row's coefficient reads go out together, ahead of the
                // FMAs that use them; at most PG rows' reads are in flight
                // (more would not fit the registers of 1024-thread blocks)
                float4 cv[D + 1];
#pragma unroll
                for (int q = 0; q <= D; ++q) cv[q] = *reinterpret_cast<const float4*>(cr + q * GF_TJ);
                if constexpr (BASE) {
                    acc[p][0] = __builtin_fmaf(r.base, wv.x, acc[p][0]);
                    acc[p][1] = __builtin_fmaf(r.base, wv.y, acc[p][1]);
                    acc[p][2] = __builtin_fmaf(r.base, wv.z, acc[p][2]);
                    acc[p][3] = __builtin_fmaf(r.base, wv.w, acc[p][3]);
                }
#pragma unroll
                for (int q = 0; q <= D; ++q) {
                    acc[p][0] = __builtin_fmaf(r.w[q], cv[q].x, acc[p][0]);
                    acc[p][1] = __builtin_fmaf(r.w[q], cv[q].y, acc[p][1]);
                    acc[p][2] = __builtin_fmaf(r.w[q], cv[q].z, acc[p][2]);
                    acc[p][3] = __builtin_fmaf(r.w[q], cv[q].w, acc[p][3]);
                }
                if (PG < 4 && p % PG == PG - 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // float32 sums over runs of at most 8 inputs (one chunk of 8, or
        // fold chunks of fewer), each folded into the float64 sums
        if ((c + 1) % fold == 0 || !more) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    accd[p][q] += (double)acc[p][q];
                    acc[p][q] = 0.0f;
                }
        }
        if (more) store(c + 1, (c + 1) & 1);
        __syncthreads();
    }
    const bool vec = (O & 3) == 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + RS * p;
        const int j = j0 + 4 * jq;
        if (b >= N || j >= O) continue;
        if (a.part) {
            double* dst = a.part + ((int64_t)slice * N + b) * O + j;
            if (vec) {
                *reinterpret_cast<double2*>(dst) = make_double2(accd[p][0], accd[p][1]);
                *reinterpret_cast<double2*>(dst + 2) = make_double2(accd[p][2], accd[p][3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (j + q < O) dst[q] = accd[p][q];
            }
        } else {
            float* dst = a.y + (int64_t)b * O + j;
            if (vec) {
                *reinterpret_cast<float4*>(dst) = make_float4((float)accd[p][0], (float)accd[p][1],
                                                              (float)accd[p][2], (float)accd[p][3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (j + q < O) dst[q] = (float)accd[p][q];
            }
        }
    }
}

// y[e] = the float64 sum over slices s = 0 .. S-1, in that order, of
// part[s n + e], rounded once to float32
__global__ void gather_sum_kernel(const double* __restrict__ part, float* __restrict__ y, int64_t n, int S) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        double v = part[e];
        for (int s = 1; s < S; ++s) v += part[s * n + e];
        y[e] = (float)v;
    }
}

// ---------------------------------------------------------------------------
// dx.  A block of 1024 threads computes 256 rows x 16 inputs: thread t takes
// input t % 16 and rows t / 16 + 64 p, p < 4, whose D + 1 basis derivatives
// and silu' it forms once.  The sum over outputs j runs in chunks of JC held
// in LDS: dy[rows][JC], the chunk's coefficients for the block's 16 inputs as
// Cs[m][ii][j] and W_base as Ws[ii][j], rows padded to JP = JC + 4 floats.
// A wave reads the coefficient rows of 16 inputs at once, each at its own
// data-dependent m; with ii the faster index and JP / 4 odd, the 16-byte
// pieces of the 16 inputs fall in distinct bank groups whatever the m (in the
// layout Cs[ii][m][j] the random m made most of these reads conflict).
// There are two chunk buffers: the next chunk is loaded into
// registers while the current one is read, with one barrier per chunk.  All
// 256 rows share a staged chunk, which keeps the coefficient staging (the
// part that grows with G) small next to the arithmetic.  With too few
// blocks to fill the GPU the outputs are split into slices whose partial dx
// are added in slice order (gather_sum_f32_kernel).
constexpr int GX_NT = 1024, GX_R = kGatherDxRows, GX_TI = kGatherDxInputs;

template <typename TS, int D, int JC>
__global__ __launch_bounds__(GX_NT) void gather_dx_kernel(GatherDxArgs a) {
    constexpr int JP = JC + 4;                       // padded LDS row (floats)
    constexpr int NPC = GX_NT / JC;                  // threads sharing one output's coefficient loads
    constexpr int MAXQ = 3;                          // ceil(K JC / 256) at the plan's K bound for JC
    constexpr int NDY = GX_R * JC / 4;               // float4 pieces of a dy chunk (<= GX_NT)
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const TS* __restrict__ x = static_cast<const TS*>(a.x);
    const TS* __restrict__ C = static_cast<const TS*>(a.C);
    const TS* __restrict__ W = static_cast<const TS*>(a.W);
    const float* __restrict__ dy = a.dy;
    const GridK g = a.g;
    const int K = g.G + D, N = a.N, I = a.I, O = a.O;
    const int dsz = GX_R * JC, csz = GX_TI * K * JP;
    const int bufsz = dsz + csz + GX_TI * JP;        // floats per chunk buffer
    const int t = threadIdx.x;

    // block -> (row block, input block), row blocks fastest on an XCD: the
    // blocks an XCD runs together share one input block's coefficients
    const int T = a.RB * a.IB;
    const int bid = blockIdx.x, nfull = T / 8, rem = T % 8, xcd = bid % 8;
    const int id = xcd * nfull + min(xcd, rem) + bid / 8;
    const int rb = id % a.RB, ibk = id / a.RB;
    const int b0 = rb * GX_R, i0 = ibk * GX_TI;
    const int nin = min(GX_TI, I - i0);
    const int slice = blockIdx.y;
    const int js = slice * a.JS, je = min(O, js + a.JS);
    const int nch = (je - js + JC - 1) / JC;

    const int il = t % GX_TI, rq = t / GX_TI;
    const int i = i0 + il;
    // per row: the LDS index of coefficient row mb = s - D clamped to
    // [0, K - D - 1] of this thread's input, and the derivative pieces
    // shifted by the clamp (as in the forward's records), then silu'
    int cb[4];
    float wd[4][D + 1], bs[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 64 * p;
        const RecD<D> r = (b < N && i < I) ? make_rec<true, D>(load_f(x, (int64_t)b * I + i), g) : zero_rec<D>();
        const int mb = clampi(r.m0, 0, K - D - 1);
        cb[p] = (mb * GX_TI + il) * JP;
#pragma unroll
        for (int q = 0; q <= D; ++q) {
            const int k = mb + q - r.m0;
            float v = 0.0f;
#pragma unroll
            for (int e = 0; e <= D; ++e) v = k == e ? r.w[e] : v;
            wd[p][q] = v;
        }
        bs[p] = a.base ? r.base : 0.0f;
    }

    // loads of one chunk: dy piece t (row t / (JC/4), columns 4 (t % (JC/4))
    // .. +3), coefficient pieces k = t / JC + NPC q of output j = t % JC's
    // run C[j, i0 .. i0+nin-1, :], and W_base[j, i0 + ii] for t < 16 JC.
    // Indices are clamped in bounds; values outside the chunk are zeroed when
    // stored.
    const bool vec = (O & 3) == 0;
    const int dyr = t / (JC / 4), dyc = 4 * (t % (JC / 4));
    const int jj = t % JC, pc = t / JC;
    const int ick = nin * K;
    float4 dp, cp[MAXQ];
    float wp;
    auto load = [&](int c) {
        const int j0 = js + c * JC;
        if (t < NDY) {
            const int b = min(b0 + dyr, N - 1), j = j0 + dyc;
            const float* row = dy + (int64_t)b * O;
            if (vec) {
                __builtin_memcpy(&dp, row + min(j, O - 4), 16);
            } else {
                dp.x = row[min(j + 0, O - 1)];
                dp.y = row[min(j + 1, O - 1)];
                dp.z = row[min(j + 2, O - 1)];
                dp.w = row[min(j + 3, O - 1)];
            }
        }
        const TS* src = C + ((int64_t)min(j0 + jj, O - 1) * I + i0) * K;
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int k = pc + NPC * q;
            if (4 * k < ick) {
                if (std::is_same<TS, float>::value && ick >= 4) {
                    __builtin_memcpy(&cp[q], reinterpret_cast<const float*>(src) + min(4 * k, ick - 4), 16);
                } else {
                    const int s = ick >= 4 ? min(4 * k, ick - 4) : 0;
                    cp[q].x = load_f(src, min(s + 0, ick - 1));
                    cp[q].y = load_f(src, min(s + 1, ick - 1));
                    cp[q].z = load_f(src, min(s + 2, ick - 1));
                    cp[q].w = load_f(src, min(s + 3, ick - 1));
                }
            }
        }
        if (t < GX_TI * JC) {
            const int wj = t / GX_TI, wi = t % GX_TI;
            wp = a.base ? load_f(W, (int64_t)min(j0 + wj, O - 1) * I + i0 + min(wi, nin - 1)) : 0.0f;
        }
    };
    auto store = [&](int c, int buf) {
        float* Ds = smem + buf * bufsz;
        float* Cs = Ds + dsz;
        float* Ws = Cs + csz;
        const int j0 = js + c * JC;
        if (t < NDY) {
            const int j = j0 + dyc;
            float4 v;
            if (vec && j < je) {
                v = dp;                                   // j .. j+3 < O, inside the slice (JS % JC == 0)
            } else {
                v.x = j + 0 < je ? dp.x : 0.0f;
                v.y = j + 1 < je ? dp.y : 0.0f;
                v.z = j + 2 < je ? dp.z : 0.0f;
                v.w = j + 3 < je ? dp.w : 0.0f;
            }
            if (b0 + dyr >= N) v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            *reinterpret_cast<float4*>(Ds + dyr * JC + dyc) = v;
        }
        const bool jok = j0 + jj < je;
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int k = pc + NPC * q;
            if (4 * k < ick) {
                // element s + e of the run is (ii, m) = divmod(s + e, K),
                // stored at (m GX_TI + ii) JP + jj; the quotient of the
                // small integer s by K is exact in float
                const int s = ick >= 4 ? min(4 * k, ick - 4) : 0;
                int ii = (int)(((float)s + 0.5f) * a.invK), m = s - ii * K;
                const float vv[4] = {cp[q].x, cp[q].y, cp[q].z, cp[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (s + e < ick) Cs[(m * GX_TI + ii) * JP + jj] = jok ? vv[e] : 0.0f;
                    if (++m == K) m = 0, ++ii;
                }
            }
        }
        if (t < GX_TI * JC) {
            const int wj = t / GX_TI, wi = t % GX_TI;
            Ws[wi * JP + wj] = (j0 + wj < je && wi < nin) ? wp : 0.0f;
        }
    };

    float Q[4][D + 2];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < D + 2; ++q) Q[p][q] = 0.0f;
    load(0);
    store(0, 0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        if (more) load(c + 1);
        const float* Ds = smem + (c & 1) * bufsz;
        const float* Cs = Ds + dsz;
        const float* Ws = Cs + csz;
        // keep the chunk's arithmetic apart from the prefetch and the stores
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
        for (int jq = 0; jq < JC; jq += 4) {
            const float4 wv = *reinterpret_cast<const float4*>(&Ws[il * JP + jq]);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float4 d = *reinterpret_cast<const float4*>(&Ds[(rq + 64 * p) * JC + jq]);
                float4 cv[D + 1];
#pragma unroll
                for (int q = 0; q <= D; ++q) cv[q] = *reinterpret_cast<const float4*>(&Cs[cb[p] + q * (GX_TI * JP) + jq]);
#pragma unroll
                for (int q = 0; q <= D; ++q) {
                    Q[p][q] = __builtin_fmaf(d.x, cv[q].x, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.y, cv[q].y, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.z, cv[q].z, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.w, cv[q].w, Q[p][q]);
                }
                Q[p][D + 1] = __builtin_fmaf(d.x, wv.x, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.y, wv.y, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.z, wv.z, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.w, wv.w, Q[p][D + 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) store(c + 1, (c + 1) & 1);
        __syncthreads();
    }
    float* out = a.part ? a.part + (int64_t)slice * N * I : a.dx;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 64 * p;
        if (b >= N || i >= I) continue;
        float v = Q[p][D + 1] * bs[p];
#pragma unroll
        for (int q = 0; q <= D; ++q) v = __builtin_fmaf(Q[p][q], wd[p][q], v);
        out[(int64_t)b * I + i] = v;
    }
}

// out[e] = the float64 sum over slices s = 0 .. S-1, in that order, of
// part[s n + e], rounded once to float32
__global__ void gather_sum_f32_kernel(const float* __restrict__ part, float* __restrict__ out, int64_t n,
                                      int S) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        double v = part[e];
        for (int s = 1; s < S; ++s) v += (double)part[s * n + e];
        out[e] = (float)v;
    }
}

// ---------------------------------------------------------------------------
// dC, dW_base.  Wave w of a block owns input i = (NT / 64) ib + w and each of
// its lanes OPL consecutive outputs j of the block's 64 OPL; every lane keeps
// the K sums dC[j, i, m] of its (j, i) pairs in registers (KMAX of them per
// output).  Rows come in chunks of 64: the block stages dy[rows][64 OPL
// outputs] in LDS, and lane l of each wave forms the span and D + 1 weights
// of row l for the wave's input.  A row's span is then the same in every lane
// of the wave, so the wave walks the spans s = 0 .. K + D - 1 as a
// compile-time loop: a ballot selects the chunk's rows whose span is s, and
// each adds dy[b, j] times its weights into the sums m = s - D .. s,
// registers named at compile time.  Rows off the grid add only their silu
// term.
// There are no atomics and no shared accumulators; the order of each sum is
// fixed by the data (rows by span, then by index).  With too few blocks to
// fill the GPU the rows are split into slices whose partial sums are added in
// slice order.  Two chunk buffers, one barrier per chunk.
template <int N0, int N1, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N0 < N1) {
        f(std::integral_constant<int, N0>());
        static_for<N0 + 1, N1>(f);
    }
}

constexpr int GC_RW = kGatherDcRecord;               // floats of a row record: w[0 .. D], silu at 7

template <int D, bool BASE, int KMAX, int OPL, int NT>
__global__ __launch_bounds__(NT) void gather_dc_kernel(GatherDcArgs a) {
    constexpr int NW = NT / 64;                      // inputs (waves) per block
    constexpr int OB = 64 * OPL;                     // outputs per block
    constexpr int DSZ = 64 * OB, WSZ = NW * 64 * GC_RW;
    constexpr int DV = DSZ / 4 / NT;                 // float4 dy pieces per thread
    typedef float vecO __attribute__((ext_vector_type(OPL)));
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const GridK g = a.g;
    const int K = g.G + D, N = a.N, I = a.I, O = a.O;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    const int T = a.IBN * a.OB;
    const int bid = blockIdx.x, nfull = T / 8, rem = T % 8, xcd = bid % 8;
    const int id = xcd * nfull + min(xcd, rem) + bid / 8;
    const int ibk = id % a.IBN, ob = id / a.IBN;
    const int i = ibk * NW + wave, j0 = ob * OB, jl = j0 + OPL * lane;
    const int slice = blockIdx.y;
    const int rs = slice * a.RS, re = min(N, rs + a.RS);
    const int nch = (re - rs + 63) / 64;
    const bool vec = (O & 3) == 0;
    const int ic = min(i, I - 1);

    float4 dp[DV];
    float xp;
    auto load = [&](int c) {
        const int r0 = rs + 64 * c;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
            const int u = t + NT * v, row = u / (OB / 4), col = 4 * (u % (OB / 4));
            const float* src = a.dy + (int64_t)min(r0 + row, N - 1) * O;
            if (vec) {
                __builtin_memcpy(&dp[v], src + min(j0 + col, O - 4), 16);
            } else {
                dp[v].x = src[min(j0 + col + 0, O - 1)];
                dp[v].y = src[min(j0 + col + 1, O - 1)];
                dp[v].z = src[min(j0 + col + 2, O - 1)];
                dp[v].w = src[min(j0 + col + 3, O - 1)];
            }
        }
        const int64_t xi = (int64_t)min(r0 + lane, N - 1) * I + ic;
        xp = a.bf16 ? load_f(static_cast<const uint16_t*>(a.x), xi) : load_f(static_cast<const float*>(a.x), xi);
    };
    int span = -1;                                   // this lane's row's span in the current chunk
    bool live = false;                               // this lane's row exists
    auto store = [&](int c, int buf) {
        float* Ds = smem + buf * (DSZ + WSZ);
        float* Wr = Ds + DSZ + wave * 64 * GC_RW;
        const int r0 = rs + 64 * c;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
            const int u = t + NT * v, row = u / (OB / 4), col = 4 * (u % (OB / 4));
            float4 d = dp[v];
            const int jc = j0 + col;
            if (!vec || jc + 3 >= O) {
                d.x = jc + 0 < O ? d.x : 0.0f;
                d.y = jc + 1 < O ? d.y : 0.0f;
                d.z = jc + 2 < O ? d.z : 0.0f;
                d.w = jc + 3 < O ? d.w : 0.0f;
            }
            if (r0 + row >= re) d = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            *reinterpret_cast<float4*>(Ds + row * OB + col) = d;
        }
        live = r0 + lane < re && i < I;
        const RecD<D> r = make_rec<false, D>(xp, g);
        span = live ? r.m0 + D : -1;
        float wr[GC_RW] = {};
#pragma unroll
        for (int q = 0; q <= D; ++q) wr[q] = r.w[q];
        wr[7] = BASE ? r.base : 0.0f;
        *reinterpret_cast<float4*>(Wr + lane * GC_RW) = make_float4(wr[0], wr[1], wr[2], wr[3]);
        *reinterpret_cast<float4*>(Wr + lane * GC_RW + 4) = make_float4(wr[4], wr[5], wr[6], wr[7]);
    };

    float acc[OPL][KMAX];
#pragma unroll
    for (int o = 0; o < OPL; ++o)
#pragma unroll
        for (int m = 0; m < KMAX; ++m) acc[o][m] = 0.0f;
    float accw[OPL];
#pragma unroll
    for (int o = 0; o < OPL; ++o) accw[o] = 0.0f;
    load(0);
    store(0, 0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        if (more) load(c + 1);
        const float* Ds = smem + (c & 1) * (DSZ + WSZ);
        const float* Wr = Ds + DSZ + wave * 64 * GC_RW;
        const int cur = span;
        // one row's dy (this lane's outputs) and weights
        auto rd = [&](int l, vecO& d, float4& w0, float4& w1) {
            d = *reinterpret_cast<const vecO*>(Ds + l * OB + OPL * lane);
            w0 = *reinterpret_cast<const float4*>(Wr + l * GC_RW);
            w1 = *reinterpret_cast<const float4*>(Wr + l * GC_RW + 4);
        };
        static_for<0, KMAX + D>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            if (s < K + D) {
                uint64_t mask = __ballot(cur == s);
                while (mask) {
                    const int l = __builtin_ctzll(mask);
                    mask &= mask - 1;
                    vecO d;
                    float4 w0, w1;
                    rd(l, d, w0, w1);
                    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int o = 0; o < OPL; ++o) {
                        static_for<0, D + 1>([&](auto rc) {
                            constexpr int r = decltype(rc)::value, m = s - D + r;
                            if constexpr (m >= 0 && m < KMAX) acc[o][m] = __builtin_fmaf(d[o], w[r], acc[o][m]);
                        });
                        if constexpr (BASE) accw[o] = __builtin_fmaf(d[o], w[7], accw[o]);
                    }
                }
            }
        });
        if constexpr (BASE) {
            // rows whose span lies off the grid: the silu term only
            uint64_t mask = __ballot(live && (cur < 0 || cur >= K + D));
            while (mask) {
                const int l = __builtin_ctzll(mask);
                mask &= mask - 1;
                const vecO d = *reinterpret_cast<const vecO*>(Ds + l * OB + OPL * lane);
                const float sv = Wr[l * GC_RW + 7];
#pragma unroll
                for (int o = 0; o < OPL; ++o) accw[o] = __builtin_fmaf(d[o], sv, accw[o]);
            }
        }
        if (more) store(c + 1, (c + 1) & 1);
        __syncthreads();
    }
    if (i < I) {
        float* dC = a.cpart ? a.cpart + (int64_t)slice * O * I * K : a.dC;
        float* dW = a.wpart ? a.wpart + (int64_t)slice * O * I : a.dW;
#pragma unroll
        for (int o = 0; o < OPL; ++o) {
            const int j = jl + o;
            if (j >= O) continue;
            if (dC) {
                float* dst = dC + ((int64_t)j * I + i) * K;
#pragma unroll
                for (int m = 0; m < KMAX; ++m)
                    if (m < K) dst[m] = acc[o][m];
            }
            if (BASE && dW) dW[(int64_t)j * I + i] = accw[o];
        }
    }
}

int grid1d(int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 8192); }

// Dynamic LDS beyond 64 KiB (gfx950 has 160 KiB per workgroup) must be requested.
template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

template <int D>
static hipError_t basis_deg_run(const GridK& g, int64_t n, int dtype, const void* x, float* B, float* dB,
                                bool tp, hipStream_t s) {
    const dim3 grid(grid1d(n * (g.G + D))), block(256);
    if (dtype == KAN_F32) {
        auto k = tp ? basis_eval_deg_kernel<float, true, D> : basis_eval_deg_kernel<float, false, D>;
        hipLaunchKernelGGL(k, grid, block, 0, s, g, n, static_cast<const float*>(x), B, dB);
    } else {
        auto k = tp ? basis_eval_deg_kernel<uint16_t, true, D> : basis_eval_deg_kernel<uint16_t, false, D>;
        hipLaunchKernelGGL(k, grid, block, 0, s, g, n, static_cast<const uint16_t*>(x), B, dB);
    }
    return hipGetLastError();
}

hipError_t launch_basis_eval(const GridK& g, int64_t n, int dtype, const void* x, float* B,
                             float* dB, bool truncated_power, int degree, hipStream_t s) {
    switch (degree) {
        case 1: return basis_deg_run<1>(g, n, dtype, x, B, dB, truncated_power, s);
        case 2: return basis_deg_run<2>(g, n, dtype, x, B, dB, truncated_power, s);
        case 4: return basis_deg_run<4>(g, n, dtype, x, B, dB, truncated_power, s);
        case 5: return basis_deg_run<5>(g, n, dtype, x, B, dB, truncated_power, s);
        default: break;
    }
    const dim3 grid(grid1d(n * (g.G + 3))), block(256);
    if (dtype == KAN_F32) {
        auto k = truncated_power ? basis_eval_kernel<float, true> : basis_eval_kernel<float, false>;
        hipLaunchKernelGGL(k, grid, block, 0, s, g, n, static_cast<const float*>(x), B, dB);
    } else {
        auto k = truncated_power ? basis_eval_kernel<uint16_t, true> : basis_eval_kernel<uint16_t, false>;
        hipLaunchKernelGGL(k, grid, block, 0, s, g, n, static_cast<const uint16_t*>(x), B, dB);
    }
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid1d((n + 7) / 8)), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid1d(n)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ---- layer launchers: degree, base branch and block size as template arguments ----
template <typename TS, int D, bool BASE, int NT>
static hipError_t gather_fwd_run(const Plan& p, const GatherFwdArgs& a, hipStream_t s) {
    constexpr int MAXQ = NT == 1024 ? 4 : 8;        // ceil(IC K / 4 / (NT / 64)) at the plan's limits
    auto k = gather_fwd_kernel<TS, D, BASE, NT, MAXQ>;
    hipError_t e = allow_lds(k, p.gf.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(p.gf.rb * p.gf.ob), (unsigned)p.gf.split), dim3(NT), p.gf.lds, s, a);
    return hipGetLastError();
}

template <typename TS, int D>
static hipError_t gather_fwd_nt(const Plan& p, const GatherFwdArgs& a, hipStream_t s) {
    if (p.gf.nt == 1024)
        return p.base ? gather_fwd_run<TS, D, true, 1024>(p, a, s) : gather_fwd_run<TS, D, false, 1024>(p, a, s);
    return p.base ? gather_fwd_run<TS, D, true, 256>(p, a, s) : gather_fwd_run<TS, D, false, 256>(p, a, s);
}

template <typename TS>
static hipError_t gather_fwd_deg(const Plan& p, const GatherFwdArgs& a, hipStream_t s) {
    switch (p.degree) {
        case 1: return gather_fwd_nt<TS, 1>(p, a, s);
        case 2: return gather_fwd_nt<TS, 2>(p, a, s);
        case 4: return gather_fwd_nt<TS, 4>(p, a, s);
        case 5: return gather_fwd_nt<TS, 5>(p, a, s);
        default: return gather_fwd_nt<TS, 3>(p, a, s);
    }
}

hipError_t launch_gather_fwd(const Plan& p, const void* x, const void* C, const void* W,
                             float* y, void* ws, hipStream_t s) {
    GatherFwdArgs a;
    a.g = p.gk;
    a.N = (int)p.N;
    a.I = (int)p.I;
    a.O = (int)p.O;
    a.IC = p.gf.ic;
    a.IS = (int)p.gf.is;
    a.RB = (int)p.gf.rb;
    a.OB = (int)p.gf.ob;
    a.x = x;
    a.C = C;
    a.W = W;
    a.y = y;
    a.part = p.gf.split > 1 ? static_cast<double*>(ws) : nullptr;
    hipError_t e = p.dtype == KAN_F32 ? gather_fwd_deg<float>(p, a, s) : gather_fwd_deg<uint16_t>(p, a, s);
    if (e != hipSuccess || p.gf.split <= 1) return e;
    const int64_t n = p.N * p.O;
    hipLaunchKernelGGL(gather_sum_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 16384)), dim3(256),
                       0, s, a.part, y, n, p.gf.split);
    return hipGetLastError();
}

template <typename TS, int D, int JC>
static hipError_t gather_dx_run(const Plan& p, const GatherDxArgs& a, hipStream_t s) {
    auto k = gather_dx_kernel<TS, D, JC>;
    hipError_t e = allow_lds(k, p.gb.lds_dx);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(p.gb.rb * p.gb.ib), (unsigned)p.gb.sx), dim3(GX_NT), p.gb.lds_dx, s, a);
    return hipGetLastError();
}

template <typename TS, int D>
static hipError_t gather_dx_jc(const Plan& p, const GatherDxArgs& a, hipStream_t s) {
    if (p.gb.jc == 16) return gather_dx_run<TS, D, 16>(p, a, s);
    if (p.gb.jc == 8) return gather_dx_run<TS, D, 8>(p, a, s);
    return gather_dx_run<TS, D, 4>(p, a, s);
}

template <typename TS>
static hipError_t gather_dx_deg(const Plan& p, const GatherDxArgs& a, hipStream_t s) {
    switch (p.degree) {
        case 1: return gather_dx_jc<TS, 1>(p, a, s);
        case 2: return gather_dx_jc<TS, 2>(p, a, s);
        case 4: return gather_dx_jc<TS, 4>(p, a, s);
        case 5: return gather_dx_jc<TS, 5>(p, a, s);
        default: return gather_dx_jc<TS, 3>(p, a, s);
    }
}

template <int D, bool BASE, int KMAX, int OPL>
static hipError_t gather_dc_run(const Plan& p, const GatherDcArgs& a, hipStream_t s) {
    constexpr int NT = KMAX * OPL <= 64 ? 1024 : 512;
    auto k = gather_dc_kernel<D, BASE, KMAX, OPL, NT>;
    hipError_t e = allow_lds(k, p.gb.lds_dc);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(p.gb.ibn * p.gb.ob), (unsigned)p.gb.sc), dim3(NT), p.gb.lds_dc, s, a);
    return hipGetLastError();
}

template <int D, bool BASE>
static hipError_t gather_dc_kmax(const Plan& p, const GatherDcArgs& a, hipStream_t s) {
    const bool two = p.gb.opl == 2;
    switch (p.gb.kmax) {
        case 16: return two ? gather_dc_run<D, BASE, 16, 2>(p, a, s) : gather_dc_run<D, BASE, 16, 1>(p, a, s);
        case 32: return two ? gather_dc_run<D, BASE, 32, 2>(p, a, s) : gather_dc_run<D, BASE, 32, 1>(p, a, s);
        case 64: return gather_dc_run<D, BASE, 64, 1>(p, a, s);
        default: return gather_dc_run<D, BASE, 132, 1>(p, a, s);
    }
}

template <int D>
static hipError_t gather_dc_base(const Plan& p, const GatherDcArgs& a, hipStream_t s) {
    return p.base ? gather_dc_kmax<D, true>(p, a, s) : gather_dc_kmax<D, false>(p, a, s);
}

static hipError_t sum_f32(const float* part, float* out, int64_t n, int S, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_sum_f32_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 16384)), dim3(256),
                       0, s, part, out, n, S);
    return hipGetLastError();
}

hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void* W,
                            const float* dy, float* dx, void* ws, hipStream_t s) {
    GatherDxArgs a;
    a.g = p.gk;
    a.N = (int)p.N;
    a.I = (int)p.I;
    a.O = (int)p.O;
    a.base = p.base;
    a.RB = (int)p.gb.rb;
    a.IB = (int)p.gb.ib;
    a.JS = (int)p.gb.js;
    a.invK = 1.0f / (float)p.K;
    a.x = x;
    a.C = C;
    a.W = W;
    a.dy = dy;
    a.dx = dx;
    a.part = p.gb.sx > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.gb.off_dxp) : nullptr;
    hipError_t e = p.dtype == KAN_F32 ? gather_dx_deg<float>(p, a, s) : gather_dx_deg<uint16_t>(p, a, s);
    if (e != hipSuccess || p.gb.sx <= 1) return e;
    return sum_f32(a.part, dx, p.N * p.I, p.gb.sx, s);
}

hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                            void* ws, hipStream_t s) {
    GatherDcArgs a;
    a.g = p.gk;
    a.N = (int)p.N;
    a.I = (int)p.I;
    a.O = (int)p.O;
    a.IBN = (int)p.gb.ibn;
    a.OB = (int)p.gb.ob;
    a.RS = (int)p.gb.rs;
    a.bf16 = p.dtype == KAN_BF16;
    a.x = x;
    a.dy = dy;
    a.dC = dC;
    a.dW = dW;
    const bool split = p.gb.sc > 1;
    char* w = static_cast<char*>(ws);
    a.cpart = split && dC ? reinterpret_cast<float*>(w + p.gb.off_dcp) : nullptr;
    a.wpart = split && dW ? reinterpret_cast<float*>(w + p.gb.off_dwp) : nullptr;
    hipError_t e;
    switch (p.degree) {
        case 1: e = gather_dc_base<1>(p, a, s); break;
        case 2: e = gather_dc_base<2>(p, a, s); break;
        case 4: e = gather_dc_base<4>(p, a, s); break;
        case 5: e = gather_dc_base<5>(p, a, s); break;
        default: e = gather_dc_base<3>(p, a, s); break;
    }
    if (e != hipSuccess || !split) return e;
    if (dC) e = sum_f32(a.cpart, dC, p.O * p.I * p.K, p.gb.sc, s);
    if (e == hipSuccess && dW) e = sum_f32(a.wpart, dW, p.O * p.I, p.gb.sc, s);
    return e;
}

}  // namespace kan
