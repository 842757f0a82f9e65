// Local 4-basis kernels on the vector ALUs (gfx950), plus the standalone basis
// evaluation, the bf16 cast and a zero fill.
//
// "Local 4-basis lookup instead of dense K-basis computation" (InKAN project
// page, "Why InKAN?"): for each (row b, input i) only the span s and the four
// pieces b0..b3 are formed; the contraction then gathers the coefficients
// C[j, i, s-3 .. s].  All arithmetic is float32 and every reduction runs in a
// fixed order without atomics.
#include <type_traits>

#include "kan_internal.h"

namespace kan {

namespace {

// Per (b, i): span-relative coefficient index base and the four weights with
// the out-of-range ones set to zero, so the inner loops can clamp the index
// and multiply unconditionally.
struct Rec {
    int m0;          // s - 3: index of the coefficient that b0 multiplies
    float w[4];      // b_r (or derivative) for m = m0 + r; 0 where m is outside [0, K-1]
    float base;      // silu(x) or silu'(x)
};

template <bool DERIV>
__device__ __forceinline__ Rec make_rec(float xv, const GridK& g) {
    Rec r;
    float u;
    const int s = span_u(xv, g, u);
    float w0, w1, w2, w3;
    if (DERIV) dpieces(u, g.scale, w0, w1, w2, w3);
    else pieces(u, w0, w1, w2, w3);
    r.m0 = s - 3;
    const int K = g.G + 3;
    r.w[0] = (r.m0 >= 0 && r.m0 < K) ? w0 : 0.0f;
    r.w[1] = (r.m0 + 1 >= 0 && r.m0 + 1 < K) ? w1 : 0.0f;
    r.w[2] = (r.m0 + 2 >= 0 && r.m0 + 2 < K) ? w2 : 0.0f;
    r.w[3] = (r.m0 + 3 >= 0 && r.m0 + 3 < K) ? w3 : 0.0f;
    r.base = DERIV ? silu_prime(xv) : silu(xv);
    return r;
}

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

// ---- basis functions of degree D != 3 (basis evaluation only) ----
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
// Forward.  Block: 64 rows x 64 outputs; thread: 4 rows x 4 consecutive outputs.
// Inputs advance in chunks of IC inputs, as many (up to 7) as keep both chunk
// buffers within 40 KB of LDS, so that 4 blocks share a CU; a chunk's
// coefficients for the 64 outputs are then at most 20 values per thread (32
// for K > 80, with one input per chunk).  They sit
// in LDS as Cs[i][m][j], so that C[j..j+3, i, m] is one 16-byte read.  LDS
// holds two chunk buffers: while one chunk is multiplied, the next chunk's
// coefficients, W_base and x are loaded into registers, and are then written
// (x as its span record) to the other buffer.  Global latency overlaps the
// arithmetic, and each chunk costs one barrier.  Each input's five-term
// partial phi_ji(x_i) is formed in float32 and added into a float64
// accumulator: a chain of KAN layers feeds y through B' of the next layer,
// which amplifies forward rounding error about tenfold, and float64 adds cost
// the same as float32 FMAs on the vector ALU.
constexpr int GF_TB = 64, GF_TJ = 64;

// A (row, input) pair of the forward chunk: the LDS index of its first
// coefficient row Cs[ii][mb][0], with mb = s - 3 clamped to [0, K - 4] so that
// rows mb .. mb + 3 all exist, and the four weights of those rows (the spline
// pieces shifted by the clamp, zero where a basis index is out of range).
struct RecF {
    int cb;
    float w[4];
    float base;
};

__device__ __forceinline__ RecF make_recf(float xv, const GridK& g, int ii, int base) {
    const Rec r = make_rec<false>(xv, g);
    const int K = g.G + 3;
    const int mb = clampi(r.m0, 0, K - 4);
    RecF f;
    f.cb = (ii * K + mb) * GF_TJ;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = mb + q - r.m0;                 // which piece multiplies row mb + q
        f.w[q] = k == 0 ? r.w[0] : k == 1 ? r.w[1] : k == 2 ? r.w[2] : k == 3 ? r.w[3] : 0.0f;
    }
    f.base = base ? r.base : 0.0f;
    return f;
}

__host__ __device__ inline int gather_fwd_ic(int K) {
    const int ic = 5120 / (GF_TJ * K + GF_TJ + GF_TB * (int)(sizeof(RecF) / 4));
    return ic < 1 ? 1 : (ic > 7 ? 7 : ic);
}
__host__ __device__ inline int gather_fwd_buf_floats(int K) {
    const int ic = gather_fwd_ic(K);
    return ic * K * GF_TJ + ic * GF_TJ + ic * GF_TB * (int)(sizeof(RecF) / 4);
}

template <typename TS, int MAXQ>
__global__ __launch_bounds__(256) void gather_fwd_kernel(GridK g, int N, int I, int O, int base,
                                                         const TS* __restrict__ x,
                                                         const TS* __restrict__ C,
                                                         const TS* __restrict__ W,
                                                         float* __restrict__ y) {
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const int K = g.G + 3;
    const int IC = gather_fwd_ic(K);
    const int ICK = IC * K;                          // coefficients of one output in a chunk
    const int csz = ICK * GF_TJ, wsz = IC * GF_TJ;
    const int bufsz = gather_fwd_buf_floats(K);      // floats per buffer: Cs, Ws, Rs
    const int t = threadIdx.x;
    const int jq = t % 16, rq = t / 16;
    const int b0 = blockIdx.x * GF_TB, j0 = blockIdx.y * GF_TJ;
    const int nch = (I + IC - 1) / IC;

    // this thread's coefficient loads: output jc = t / 4 of the tile, and of
    // that output's ICK chunk coefficients (rem = ii * K + m, contiguous in
    // C) those with rem = t % 4 + 4 q
    const int jc = t >> 2, rc = t & 3;
    const int nq = (ICK + 3) / 4;                    // <= MAXQ
    // W_base and x: the 64 IC (output or row, input) pairs of a chunk, pair
    // u = t + 256 v (v < 2, as IC <= 7) at pair index pj = u / IC, pi = u % IC
    int pj[2], pi[2];
    bool has_pair[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int u = t + 256 * v;
        has_pair[v] = u < IC * 64;
        pj[v] = u / IC;
        pi[v] = u % IC;
    }

    // Loads are issued unconditionally from addresses clamped in bounds (a
    // guarded load into a register that was zeroed first makes the compiler
    // wait for every earlier load); invalid values are zeroed when stored.
    float cp[std::is_same<TS, float>::value ? 1 : MAXQ];
    constexpr int NV = (MAXQ + 3) / 4;               // float32: 16-byte pieces per thread
    float4 cp4[std::is_same<TS, float>::value ? NV : 1];
    const int nv = (ICK + 15) / 16;
    float wp[2], xp[2];
    const bool jc_ok = j0 + jc < O;
    auto load = [&](int c) {
        const int i0 = c * IC, nic = min(IC, I - i0);
        // row of output j0 + jc from input i0 on (output 0 when the output
        // does not exist); indices past the chunk's last input are clamped
        const TS* row = C + (jc_ok ? ((int64_t)(j0 + jc) * I + i0) * K : 0);
        const int last = jc_ok ? nic * K - 1 : 0;
        if constexpr (std::is_same<TS, float>::value) {
            // 16-byte pieces k = rc + 4 q of the output's chunk row, each
            // clamped to start inside it (a clamped piece repeats values)
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int s = jc_ok ? min(4 * (rc + 4 * q), last - 3) : 0;
                if (q < nv) __builtin_memcpy(&cp4[q], row + s, 16);
            }
        } else {
#pragma unroll
            for (int q = 0; q < MAXQ; ++q)
                if (q < nq) cp[q] = load_f(row, min(rc + 4 * q, last));
        }
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const bool okw = has_pair[v] && base && j0 + pj[v] < O && pi[v] < nic;
            const bool okx = has_pair[v] && b0 + pj[v] < N && pi[v] < nic;
            wp[v] = load_f(W ? W : x, okw ? (int64_t)(j0 + pj[v]) * I + i0 + pi[v] : 0);
            xp[v] = load_f(x, okx ? (int64_t)(b0 + pj[v]) * I + i0 + pi[v] : 0);
            wp[v] = okw ? wp[v] : 0.0f;
        }
    };
    auto store = [&](int c, int buf) {
        float* Cs = smem + buf * bufsz;
        float* Ws = Cs + csz;
        RecF* Rs = reinterpret_cast<RecF*>(Ws + wsz);
        const int i0 = c * IC, nic = min(IC, I - i0);
        const int lim = jc_ok ? nic * K : 0;         // valid coefficients of this output
        if constexpr (std::is_same<TS, float>::value) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int s = jc_ok ? min(4 * (rc + 4 * q), lim - 4) : 0;
                if (q < nv && jc_ok) {
                    Cs[(s + 0) * GF_TJ + jc] = cp4[q].x;
                    Cs[(s + 1) * GF_TJ + jc] = cp4[q].y;
                    Cs[(s + 2) * GF_TJ + jc] = cp4[q].z;
                    Cs[(s + 3) * GF_TJ + jc] = cp4[q].w;
                }
            }
            for (int rem = lim + rc; rem < ICK; rem += 4) Cs[rem * GF_TJ + jc] = 0.0f;
        } else {
#pragma unroll
            for (int q = 0; q < MAXQ; ++q) {
                const int rem = rc + 4 * q;
                if (q < nq && rem < ICK) Cs[rem * GF_TJ + jc] = rem < lim ? cp[q] : 0.0f;
            }
        }
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            if (!has_pair[v]) continue;
            Ws[pi[v] * GF_TJ + pj[v]] = wp[v];
            RecF r;
            if (b0 + pj[v] < N && pi[v] < nic) {
                r = make_recf(xp[v], g, pi[v], base);
            } else {
                r.cb = pi[v] * K * GF_TJ;
                r.w[0] = r.w[1] = r.w[2] = r.w[3] = 0.0f;
                r.base = 0.0f;
            }
            Rs[pi[v] * GF_TB + pj[v]] = r;
        }
    };

    double acc[4][4] = {};
    load(0);
    store(0, 0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        if (more) load(c + 1);
        const float* Cs = smem + (c & 1) * bufsz;
        const float* Ws = Cs + csz;
        const RecF* Rs = reinterpret_cast<const RecF*>(Ws + wsz);
        const int nic = min(IC, I - c * IC);
        for (int ii = 0; ii < nic; ++ii) {
            const float4 wv = *reinterpret_cast<const float4*>(&Ws[ii * GF_TJ + 4 * jq]);
            RecF rr[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) rr[p] = Rs[ii * GF_TB + rq + 16 * p];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const RecF& r = rr[p];
                const float* crow = Cs + r.cb + 4 * jq;
                // the row's four coefficient reads go out together, ahead of
                // the FMAs that use them
                float4 cv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cv[q] = *reinterpret_cast<const float4*>(crow + q * GF_TJ);
                float a0 = r.base * wv.x, a1 = r.base * wv.y, a2 = r.base * wv.z, a3 = r.base * wv.w;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    a0 = __builtin_fmaf(r.w[q], cv[q].x, a0);
                    a1 = __builtin_fmaf(r.w[q], cv[q].y, a1);
                    a2 = __builtin_fmaf(r.w[q], cv[q].z, a2);
                    a3 = __builtin_fmaf(r.w[q], cv[q].w, a3);
                }
                acc[p][0] += (double)a0;
                acc[p][1] += (double)a1;
                acc[p][2] += (double)a2;
                acc[p][3] += (double)a3;
            }
        }
        if (more) store(c + 1, (c + 1) & 1);
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 16 * p;
        if (b >= N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = j0 + 4 * jq + q;
            if (j < O) y[(int64_t)b * O + j] = (float)acc[p][q];
        }
    }
}

// ---------------------------------------------------------------------------
// dx.  Block: 64 rows x 16 inputs; thread: 4 rows x 1 input.  The reduction
// runs over outputs j in chunks of 16 with dy and C staged in LDS.
constexpr int GX_TB = 64, GX_TI = 16, GX_JC = 16;

template <typename TS>
__global__ __launch_bounds__(256) void gather_dx_kernel(GridK g, int N, int I, int O, int base,
                                                        const TS* __restrict__ x,
                                                        const TS* __restrict__ C,
                                                        const TS* __restrict__ W,
                                                        const float* __restrict__ dy,
                                                        float* __restrict__ dx) {
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const int K = g.G + 3;
    float* Ds = smem;                               // [TB][JC]
    float* Cs = Ds + GX_TB * GX_JC;                  // [TI][K][JC]
    float* Ws = Cs + GX_TI * K * GX_JC;              // [TI][JC]

    const int t = threadIdx.x;
    const int il = t % GX_TI, rq = t / GX_TI;
    const int b0 = blockIdx.x * GX_TB, i0 = blockIdx.y * GX_TI;
    const int i = i0 + il;
    Rec rec[4];
    int mi[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 16 * p;
        if (b < N && i < I) {
            rec[p] = make_rec<true>(load_f(x, (int64_t)b * I + i), g);
            if (!base) rec[p].base = 0.0f;
        } else {
            rec[p].m0 = 0;
            rec[p].w[0] = rec[p].w[1] = rec[p].w[2] = rec[p].w[3] = 0.0f;
            rec[p].base = 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) mi[p][q] = clampi(rec[p].m0 + q, 0, K - 1);
    }
    float Q[4][5] = {};
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
                for (int q = 0; q < 4; ++q) {
                    const float4 c = *reinterpret_cast<const float4*>(&Cs[(il * K + mi[p][q]) * GX_JC + jj]);
                    Q[p][q] = __builtin_fmaf(d.x, c.x, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.y, c.y, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.z, c.z, Q[p][q]);
                    Q[p][q] = __builtin_fmaf(d.w, c.w, Q[p][q]);
                }
                Q[p][4] = __builtin_fmaf(d.x, wv.x, Q[p][4]);
                Q[p][4] = __builtin_fmaf(d.y, wv.y, Q[p][4]);
                Q[p][4] = __builtin_fmaf(d.z, wv.z, Q[p][4]);
                Q[p][4] = __builtin_fmaf(d.w, wv.w, Q[p][4]);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int b = b0 + rq + 16 * p;
        if (b >= N || i >= I) continue;
        float v = Q[p][4] * rec[p].base;
#pragma unroll
        for (int q = 0; q < 4; ++q) v = __builtin_fmaf(Q[p][q], rec[p].w[q], v);
        dx[(int64_t)b * I + i] = v;
    }
}

// ---------------------------------------------------------------------------
// dC, dW_base.  Block owns 16 inputs x 16 outputs and sweeps every row in a
// fixed order; thread (i, j) keeps its K spline accumulators in a private LDS
// column (no other thread touches them, so there is no atomic and the sum
// order is the row order).
constexpr int GC_TI = 16, GC_TJ = 16, GC_RB = 64;

template <typename TS>
__global__ __launch_bounds__(256) void gather_dc_kernel(GridK g, int N, int I, int O, int base,
                                                        const TS* __restrict__ x,
                                                        const float* __restrict__ dy,
                                                        float* __restrict__ dC,
                                                        float* __restrict__ dW) {
    extern __shared__ float4 smem4[];
    float* smem = reinterpret_cast<float*>(smem4);
    const int K = g.G + 3;
    float* Acc = smem;                                // [K][256]
    float* Ds = Acc + K * 256;                        // [RB][TJ]
    Rec* Rs = reinterpret_cast<Rec*>(Ds + GC_RB * GC_TJ);  // [RB][TI]

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
            Rec r;
            if (b < N && i < I) {
                r = make_rec<false>(load_f(x, (int64_t)b * I + i), g);
            } else {
                r.m0 = 0;
                r.w[0] = r.w[1] = r.w[2] = r.w[3] = 0.0f;
                r.base = 0.0f;
            }
            Rs[bb * GC_TI + ii] = r;
        }
        __syncthreads();
        const int nb = min(GC_RB, N - r0);
        for (int bb = 0; bb < nb; ++bb) {
            const float d = Ds[bb * GC_TJ + jl];
            const Rec r = Rs[bb * GC_TI + il];
            accw = __builtin_fmaf(d, r.base, accw);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
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

template <typename TS, int MAXQ>
static hipError_t gather_fwd_run(const Plan& p, const void* x, const void* C, const void* W, float* y,
                                 hipStream_t s) {
    const size_t lds = (size_t)2 * gather_fwd_buf_floats(p.K) * 4;   // two chunk buffers
    dim3 grid((unsigned)((p.N + GF_TB - 1) / GF_TB), (unsigned)((p.O + GF_TJ - 1) / GF_TJ));
    hipError_t e = allow_lds(gather_fwd_kernel<TS, MAXQ>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gather_fwd_kernel<TS, MAXQ>), grid, dim3(256), lds, s, p.gk, (int)p.N, (int)p.I,
                       (int)p.O, p.base, static_cast<const TS*>(x), static_cast<const TS*>(C),
                       static_cast<const TS*>(W), y);
    return hipGetLastError();
}

// prefetch registers per thread: ceil(64 IC K / 256) coefficients
template <typename TS>
static hipError_t gather_fwd_t(const Plan& p, const void* x, const void* C, const void* W,
                               float* y, hipStream_t s) {
    const int nq = (gather_fwd_ic(p.K) * p.K * GF_TJ + 255) / 256;
    if (nq <= 20) return gather_fwd_run<TS, 20>(p, x, C, W, y, s);
    return gather_fwd_run<TS, 32>(p, x, C, W, y, s);
}

template <typename TS>
static hipError_t gather_dx_t(const Plan& p, const void* x, const void* C, const void* W,
                              const float* dy, float* dx, hipStream_t s) {
    const size_t lds = (size_t)(GX_TB * GX_JC + GX_TI * p.K * GX_JC + GX_TI * GX_JC) * 4;
    dim3 grid((unsigned)((p.N + GX_TB - 1) / GX_TB), (unsigned)((p.I + GX_TI - 1) / GX_TI));
    hipError_t e = allow_lds(gather_dx_kernel<TS>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gather_dx_kernel<TS>, grid, dim3(256), lds, s, p.gk, (int)p.N, (int)p.I,
                       (int)p.O, p.base, static_cast<const TS*>(x), static_cast<const TS*>(C),
                       static_cast<const TS*>(W), dy, dx);
    return hipGetLastError();
}

template <typename TS>
static hipError_t gather_dc_t(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                              hipStream_t s) {
    const size_t lds = (size_t)(p.K * 256 + GC_RB * GC_TJ) * 4 + GC_RB * GC_TI * sizeof(Rec);
    dim3 grid((unsigned)((p.I + GC_TI - 1) / GC_TI), (unsigned)((p.O + GC_TJ - 1) / GC_TJ));
    hipError_t e = allow_lds(gather_dc_kernel<TS>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gather_dc_kernel<TS>, grid, dim3(256), lds, s, p.gk, (int)p.N, (int)p.I,
                       (int)p.O, p.base, static_cast<const TS*>(x), dy, dC, dW);
    return hipGetLastError();
}

hipError_t launch_gather_fwd(const Plan& p, const void* x, const void* C, const void* W,
                             float* y, hipStream_t s) {
    return p.dtype == KAN_F32 ? gather_fwd_t<float>(p, x, C, W, y, s)
                              : gather_fwd_t<uint16_t>(p, x, C, W, y, s);
}
hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void* W,
                            const float* dy, float* dx, hipStream_t s) {
    return p.dtype == KAN_F32 ? gather_dx_t<float>(p, x, C, W, dy, dx, s)
                              : gather_dx_t<uint16_t>(p, x, C, W, dy, dx, s);
}
hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                            hipStream_t s) {
    return p.dtype == KAN_F32 ? gather_dc_t<float>(p, x, dy, dC, dW, s)
                              : gather_dc_t<uint16_t>(p, x, dy, dC, dW, s);
}

}  // namespace kan
