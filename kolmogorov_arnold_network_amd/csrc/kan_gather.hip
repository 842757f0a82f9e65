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

__global__ void cast_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
    for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x)
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
// - A thread's sums over one chunk are float32; each chunk's sum is added
//   into a float64 accumulator.  In a chain of layers the next layer's B'
//   amplifies forward rounding about tenfold, so the long sum over inputs
//   is kept out of float32.
// - All R rows of the block share one staged chunk, so the coefficient
//   traffic per row, the part of the work that grows with G, falls as R
//   grows.
// - With too few blocks to fill the GPU the inputs are split into slices.
//   Each slice writes float64 partial outputs, which gather_sum_kernel adds
//   in slice order.
constexpr int GF_TJ = 64;

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
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                accd[p][q] += (double)acc[p][q];
                acc[p][q] = 0.0f;
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
// dx.  Block: 64 rows x 16 inputs; thread: 4 rows x 1 input.  The reduction
// runs over outputs j in chunks of 16 with dy and C staged in LDS.
constexpr int GX_TB = 64, GX_TI = 16, GX_JC = 16;

template <typename TS, int D>
__global__ __launch_bounds__(256) void gather_dx_kernel(GridK g, int N, int I, int O, int base,
                                                        const TS* __restrict__ x,
                                                        const TS* __restrict__ C,
                                                        const TS* __restrict__ W,
                                                        const float* __restrict__ dy,
                                                        float* __restrict__ dx) {
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const int K = g.G + D;
    float* Ds = smem;                               // [TB][JC]
    float* Cs = Ds + GX_TB * GX_JC;                  // [TI][K][JC]
    float* Ws = Cs + GX_TI * K * GX_JC;              // [TI][JC]

    const int t = threadIdx.x;
    const int il = t % GX_TI, rq = t / GX_TI;
    const int b0 = blockIdx.x * GX_TB, i0 = blockIdx.y * GX_TI;
    const int i = i0 + il;
    RecD<D> rec[4];
    int mi[4][D + 1];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 16 * p;
        if (b < N && i < I) {
            rec[p] = make_rec<true, D>(load_f(x, (int64_t)b * I + i), g);
            if (!base) rec[p].base = 0.0f;
        } else {
            rec[p] = zero_rec<D>();
        }
#pragma unroll
        for (int q = 0; q <= D; ++q) mi[p][q] = clampi(rec[p].m0 + q, 0, K - 1);
    }
    float Q[4][D + 2];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < D + 2; ++q) Q[p][q] = 0.0f;
    for (int jc = 0; jc < O; jc += GX_JC) {
        __syncthreads();
        for (int e = t; e < GX_TB * GX_JC; e += 256) {
            const int bb = e / GX_JC, jj = e % GX_JC;
            const int b = b0 + bb, j = jc + jj;
            Ds[bb * GX_JC + jj] = (b < N && j < O) ? dy[(int64_t)b * O + j] : 0.0f;
        }
        for (int e = t; e < GX_JC * GX_TI * K; e += 256) {
            const int jj = e / (GX_TI * K), rem = e % (GX_TI * K);
            const int ii = rem / K, m = rem % K;
            const int j = jc + jj, ig = i0 + ii;
            Cs[(ii * K + m) * GX_JC + jj] =
                (j < O && ig < I) ? load_f(C, ((int64_t)j * I + ig) * K + m) : 0.0f;
        }
        for (int e = t; e < GX_JC * GX_TI; e += 256) {
            const int jj = e / GX_TI, ii = e % GX_TI;
            const int j = jc + jj, ig = i0 + ii;
            Ws[ii * GX_JC + jj] = (base && j < O && ig < I) ? load_f(W, (int64_t)j * I + ig) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < GX_JC; jj += 4) {
            const float4 wv = *reinterpret_cast<const float4*>(&Ws[il * GX_JC + jj]);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float4 d = *reinterpret_cast<const float4*>(&Ds[(rq + 16 * p) * GX_JC + jj]);
#pragma unroll
                for (int q = 0; q <= D; ++q) {
                    const float4 c = *reinterpret_cast<const float4*>(&Cs[(il * K + mi[p][q]) * GX_JC + jj]);
                    Q[p][q] = __builtin_fmaf(d.x, c.x, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.y, c.y, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.z, c.z, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.w, c.w, Q[p][q]);
                }
                Q[p][D + 1] = __builtin_fmaf(d.x, wv.x, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.y, wv.y, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.z, wv.z, Q[p][D + 1]);
                Q[p][D + 1] = __builtin_fmaf(d.w, wv.w, Q[p][D + 1]);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 16 * p;
        if (b >= N || i >= I) continue;
        float v = Q[p][D + 1] * rec[p].base;
#pragma unroll
        for (int q = 0; q <= D; ++q) v = __builtin_fmaf(Q[p][q], rec[p].w[q], v);
        dx[(int64_t)b * I + i] = v;
    }
}

// ---------------------------------------------------------------------------
// dC, dW_base.  Block owns 16 inputs x 16 outputs and sweeps every row in a
// fixed order; thread (i, j) keeps its K spline accumulators in a private LDS
// column (no other thread touches them, so there is no atomic and the sum
// order is the row order).  Rows are staged GC_RB at a time (32 above degree
// 3, whose larger records would push G = 125 past the 160 KB of LDS).
constexpr int GC_TI = 16, GC_TJ = 16;
template <int D> constexpr int gc_rb() { return D > 3 ? 32 : 64; }

template <typename TS, int D>
__global__ __launch_bounds__(256) void gather_dc_kernel(GridK g, int N, int I, int O, int base,
                                                        const TS* __restrict__ x,
                                                        const float* __restrict__ dy,
                                                        float* __restrict__ dC,
                                                        float* __restrict__ dW) {
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const int K = g.G + D;
    float* Acc = smem;                                // [K][256]
    float* Ds = Acc + K * 256;                        // [RB][TJ]
    constexpr int GC_RB = gc_rb<D>();
    RecD<D>* Rs = reinterpret_cast<RecD<D>*>(Ds + GC_RB * GC_TJ);  // [RB][TI]

    const int t = threadIdx.x;
    const int il = t % GC_TI, jl = t / GC_TI;
    const int i0 = blockIdx.x * GC_TI, j0 = blockIdx.y * GC_TJ;
    for (int m = 0; m < K; ++m) Acc[m * 256 + t] = 0.0f;
    float accw = 0.0f;
    for (int r0 = 0; r0 < N; r0 += GC_RB) {
        __syncthreads();
        for (int e = t; e < GC_RB * GC_TJ; e += 256) {
            const int bb = e / GC_TJ, jj = e % GC_TJ;
            const int b = r0 + bb, j = j0 + jj;
            Ds[bb * GC_TJ + jj] = (b < N && j < O) ? dy[(int64_t)b * O + j] : 0.0f;
        }
        for (int e = t; e < GC_RB * GC_TI; e += 256) {
            const int bb = e / GC_TI, ii = e % GC_TI;
            const int b = r0 + bb, i = i0 + ii;
            Rs[bb * GC_TI + ii] = (b < N && i < I) ? make_rec<false, D>(load_f(x, (int64_t)b * I + i), g)
                                                   : zero_rec<D>();
        }
        __syncthreads();
        const int nb = min(GC_RB, N - r0);
        for (int bb = 0; bb < nb; ++bb) {
            const float d = Ds[bb * GC_TJ + jl];
            const RecD<D> r = Rs[bb * GC_TI + il];
            accw = __builtin_fmaf(d, r.base, accw);
#pragma unroll
            for (int q = 0; q <= D; ++q) {
                const int m = clampi(r.m0 + q, 0, K - 1);
                Acc[m * 256 + t] = __builtin_fmaf(d, r.w[q], Acc[m * 256 + t]);
            }
        }
    }
    const int i = i0 + il, j = j0 + jl;
    if (i < I && j < O) {
        if (dC)
            for (int m = 0; m < K; ++m) dC[((int64_t)j * I + i) * K + m] = Acc[m * 256 + t];
        if (dW && base) dW[(int64_t)j * I + i] = accw;
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

GatherFwdPlan gather_fwd_plan(int64_t N, int64_t I, int64_t O, int K, int D, int base) {
    GatherFwdPlan q;
    const int64_t ob = (O + GF_TJ - 1) / GF_TJ;
    // 256-row blocks of 1024 threads when they still make 64 or more blocks
    // (or when K is large, where staging dominates); 64-row blocks of 256
    // threads for small batches
    q.nt = ((N + 255) / 256 * ob >= 64 || K > 32) ? 1024 : 256;
    const int R = q.nt / 4;
    const int rw = ((D + 3) + 1) & ~1;                       // words of a span record
    const int64_t per_in = (int64_t)GF_TJ * K + (base ? GF_TJ : 0) + (int64_t)R * rw;
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
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid1d(n)), dim3(256), 0, s, in, out, n);
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

template <typename TS, int D>
static hipError_t gather_dx_run(const Plan& p, const void* x, const void* C, const void* W,
                                const float* dy, float* dx, hipStream_t s) {
    const size_t lds = (size_t)(GX_TB * GX_JC + GX_TI * p.K * GX_JC + GX_TI * GX_JC) * 4;
    dim3 grid((unsigned)((p.N + GX_TB - 1) / GX_TB), (unsigned)((p.I + GX_TI - 1) / GX_TI));
    hipError_t e = allow_lds(gather_dx_kernel<TS, D>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gather_dx_kernel<TS, D>), grid, dim3(256), lds, s, p.gk, (int)p.N, (int)p.I,
                       (int)p.O, p.base, static_cast<const TS*>(x), static_cast<const TS*>(C),
                       static_cast<const TS*>(W), dy, dx);
    return hipGetLastError();
}

template <typename TS, int D>
static hipError_t gather_dc_run(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                                hipStream_t s) {
    constexpr int GC_RB = gc_rb<D>();
    const size_t lds = (size_t)(p.K * 256 + GC_RB * GC_TJ) * 4 + GC_RB * GC_TI * sizeof(RecD<D>);
    dim3 grid((unsigned)((p.I + GC_TI - 1) / GC_TI), (unsigned)((p.O + GC_TJ - 1) / GC_TJ));
    hipError_t e = allow_lds(gather_dc_kernel<TS, D>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gather_dc_kernel<TS, D>), grid, dim3(256), lds, s, p.gk, (int)p.N, (int)p.I,
                       (int)p.O, p.base, static_cast<const TS*>(x), dy, dC, dW);
    return hipGetLastError();
}

template <typename TS>
static hipError_t gather_dx_deg(const Plan& p, const void* x, const void* C, const void* W,
                                const float* dy, float* dx, hipStream_t s) {
    switch (p.degree) {
        case 1: return gather_dx_run<TS, 1>(p, x, C, W, dy, dx, s);
        case 2: return gather_dx_run<TS, 2>(p, x, C, W, dy, dx, s);
        case 4: return gather_dx_run<TS, 4>(p, x, C, W, dy, dx, s);
        case 5: return gather_dx_run<TS, 5>(p, x, C, W, dy, dx, s);
        default: return gather_dx_run<TS, 3>(p, x, C, W, dy, dx, s);
    }
}

template <typename TS>
static hipError_t gather_dc_deg(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                                hipStream_t s) {
    switch (p.degree) {
        case 1: return gather_dc_run<TS, 1>(p, x, dy, dC, dW, s);
        case 2: return gather_dc_run<TS, 2>(p, x, dy, dC, dW, s);
        case 4: return gather_dc_run<TS, 4>(p, x, dy, dC, dW, s);
        case 5: return gather_dc_run<TS, 5>(p, x, dy, dC, dW, s);
        default: return gather_dc_run<TS, 3>(p, x, dy, dC, dW, s);
    }
}

hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void* W,
                            const float* dy, float* dx, hipStream_t s) {
    return p.dtype == KAN_F32 ? gather_dx_deg<float>(p, x, C, W, dy, dx, s)
                              : gather_dx_deg<uint16_t>(p, x, C, W, dy, dx, s);
}
hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                            hipStream_t s) {
    return p.dtype == KAN_F32 ? gather_dc_deg<float>(p, x, dy, dC, dW, s)
                              : gather_dc_deg<uint16_t>(p, x, dy, dC, dW, s);
}

}  // namespace kan
