// Per-channel (grouped) spline activation on gfx950:
//
//     y[b, i]  = sum_m C[g(i), m] * B_m(x[b, i]),          g(i) = i * groups / I
//     dx[b, i] = dy[b, i] * sum_m C[g(i), m] * B'_m(x[b, i])
//     dC[g, m] = sum_b sum_{i in g} dy[b, i] * B_m(x[b, i])
//
// the element-wise form of the KAN edge function, one learned spline per
// group of consecutive channels (InKAN project page: per-coordinate spline
// curves; FlashKAT abstract: grouped KAN activations, whose training is slowed
// by atomic accumulation of the coefficient gradient).  Each element is read
// and written once, so the floor is HBM traffic; with 64-lane float32 ALUs the
// per-element instruction count is the other limit, and the kernels keep it
// small:
//
// - On knot span s (local coordinate u) the spline is one cubic,
//   sum_r C[s-3+r] b_r(u) = a0 + a1 u + a2 u^2 + a3 u^3 (the b_r are the four
//   uniform cubic pieces).  A block tabulates (a0..a3) per span of the groups
//   it meets in LDS, so an element costs one 16-byte LDS read and a Horner
//   step, and dx the derivative cubic (a1 + 2 a2 u + 3 a3 u^2) / h.
// - dC is reduced without atomics: every thread adds dy * b_r(u) into its own
//   LDS column, whose rows are padded by 3 on each side so that the 4 rows of
//   a span need no bounds checks; fixed-order passes then add the columns of
//   the block's row waves, the per-chunk partials, and a group's channels.
//
// Grids with many groups and a large G, whose tables would not fit in LDS,
// take a plain path: the four pieces and coefficients read from memory.
#include <type_traits>

#include "kan_internal.h"

namespace kan {

namespace {

constexpr int GP_C = kGroupChannels;    // channels per block (one per lane)
constexpr int GP_W = kGroupWaves;       // row waves per block
constexpr int GP_T = GP_C * GP_W;       // threads per block
constexpr int GP_UF = kGroupRowsFwd;    // rows whose loads a forward thread issues together
constexpr int GP_UB = kGroupRowsBwd;    // the same, backward
constexpr size_t kTabLimit = 32 * 1024; // LDS bytes for the per-span table

// p[i] for a wave-uniform row base p and a lane's channel i, as a 32-bit
// unsigned byte offset from p (the backward's global loads and stores; the
// buffer form below saves address arithmetic but measured slower there)
template <typename T>
__device__ __forceinline__ T& at(T* p, int i) {
    using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
    return *reinterpret_cast<T*>(reinterpret_cast<B*>(p) + (uint32_t)i * (uint32_t)sizeof(T));
}
// streamed (non-temporal) loads and stores of that form
__device__ __forceinline__ float load_at(const float* p, int i) { return __builtin_nontemporal_load(&at(p, i)); }
__device__ __forceinline__ float load_at(const uint16_t* p, int i) {
    return __uint_as_float(((uint32_t)__builtin_nontemporal_load(&at(p, i))) << 16);
}

// Raw buffer access to one row of `bytes` bytes at a wave-uniform base: the
// resource is built in scalar registers, a lane supplies only its 32-bit
// byte offset, and offsets past the row read 0 / write nothing.  The third
// resource word is the gfx9-family raw-buffer format.  Every element is
// touched once, so loads and stores carry the non-temporal cache policy
// (kNT); measured on g1, it took the forward from 4.6 to 5.3 TB/s.
constexpr int kNT = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ float row_load(const float* row, int I, int i) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row_rsrc(row, I * 4), i * 4, 0, kNT));
}
__device__ __forceinline__ float row_load(const uint16_t* row, int I, int i) {
    return __uint_as_float(((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(row_rsrc(row, I * 2), i * 2, 0, kNT))
                           << 16);
}
__device__ __forceinline__ void row_store(float* row, int I, int i, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), row_rsrc(row, I * 4), i * 4, 0, kNT);
}

__device__ __forceinline__ int group_of(int i, int I, int groups) {
    return (int)(((int64_t)i * groups) / I);
}

// Polynomial coefficients of the spline on span s of group g (C rows of K;
// m outside [0, K) are zero): forward (a0, a1, a2, a3), or backward the
// derivative's (a1, 2 a2, 3 a3) / h.
template <typename TS>
__device__ __forceinline__ float4 span_cubic(const TS* C, int g, int s, int K, float scale, bool deriv) {
    float c[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = s - 3 + r;
        c[r] = (m >= 0 && m < K) ? load_f(C, (int64_t)g * K + m) : 0.0f;
    }
    const float a0 = (c[0] + 4.0f * c[1] + c[2]) * (1.0f / 6.0f);
    const float a1 = (c[2] - c[0]) * 0.5f;
    const float a2 = (c[0] - 2.0f * c[1] + c[2]) * 0.5f;
    const float a3 = (c[3] - c[0] + 3.0f * (c[1] - c[2])) * (1.0f / 6.0f);
    return deriv ? make_float4(a1 * scale, 2.0f * a2 * scale, 3.0f * a3 * scale, 0.0f)
                 : make_float4(a0, a1, a2, a3);
}

// The groups met by the block's channels, and the table of their spans.
struct BlockGroups {
    int g0, n;
};
__device__ __forceinline__ BlockGroups block_groups(int I, int groups) {
    const int c0 = blockIdx.x * GP_C, c1 = min(c0 + GP_C, I) - 1;
    BlockGroups bg;
    bg.g0 = group_of(c0, I, groups);
    bg.n = group_of(c1, I, groups) - bg.g0 + 1;
    return bg;
}

template <typename TS>
__device__ __forceinline__ void build_table(float4* tab, const TS* C, const BlockGroups& bg, const GridK& g,
                                            bool deriv) {
    const int S = g.G + 6, K = g.G + 3;
    for (int e = threadIdx.x; e < bg.n * S; e += GP_T) {
        const int gl = e / S;
        tab[e] = span_cubic(C, bg.g0 + gl, e - gl * S, K, g.scale, deriv);
    }
}

// Forward.  Block (bx, by): channels bx*64 + lane, rows by*R .. by*R+R-1, of
// which wave w takes rows w, w+4, ...
template <typename TS, bool TAB>
__global__ void __launch_bounds__(GP_T, 8) grouped_fwd_kernel(GridK g, int N, int I, int groups, int R,
                                                              const TS* __restrict__ x,
                                                              const TS* __restrict__ C,
                                                              float* __restrict__ y) {
    extern __shared__ float4 tab[];
    const int K = g.G + 3, S = g.G + 6;
    // the row wave index is uniform across a wave: rows, and so row base
    // addresses, live in scalar registers, and a lane adds only its channel
    const int lane = threadIdx.x & (GP_C - 1), w = __builtin_amdgcn_readfirstlane(threadIdx.x / GP_C);
    const int i = blockIdx.x * GP_C + lane;
    const BlockGroups bg = block_groups(I, groups);
    if (TAB) {
        build_table(tab, C, bg, g, false);
        __syncthreads();
    }
    if (i >= I) return;                                // no barrier below
    const int gi = group_of(i, I, groups);
    const float4* t = tab + (gi - bg.g0) * S;
    const TS* c = C + (int64_t)gi * K;
    const int r0 = blockIdx.y * R, r1 = min(r0 + R, N);
    for (int b = r0 + w; b < r1; b += GP_W * GP_UF) {
        float xv[GP_UF];
#pragma unroll
        for (int q = 0; q < GP_UF; ++q) xv[q] = row_load(x + (int64_t)min(b + q * GP_W, r1 - 1) * I, I, i);
        // every row of the batch is computed (rows past the chunk repeat its
        // last row) and only the stores are predicated, so that the loads are
        // all issued before the first use
#pragma unroll
        for (int q = 0; q < GP_UF; ++q) {
            const int row = b + q * GP_W;
            float u;
            const int s = span_u(xv[q], g, u);
            float v;
            if (TAB) {
                const bool in = (unsigned)s < (unsigned)S;
                const float4 a = t[in ? s : 0];
                v = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(a.w, u, a.z), u, a.y), u, a.x);
                v = in ? v : 0.0f;
            } else {
                float p[4];
                pieces(u, p[0], p[1], p[2], p[3]);
                v = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = s - 3 + r;
                    if (m >= 0 && m < K) v = __builtin_fmaf(load_f(c, m), p[r], v);
                }
            }
            // a row past the chunk stores through a zero-size resource, which
            // drops the write: no branch, so no load is sunk behind a store
            row_store(y + (int64_t)min(row, r1 - 1) * I, row < r1 ? I : 0, i, v);
        }
    }
}

// Forward with two adjacent channels per lane (I even): one 4-byte (bf16)
// or 8-byte (float32) load and one 8-byte store per row, so a wave moves
// twice the bytes per memory instruction.  Block: 128 channels, 4 row waves.
constexpr int GP_C2 = 2 * GP_C;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void row_load2(const uint16_t* row, int I, int i, float& a, float& b) {
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(row_rsrc(row, I * 2), i * 2, 0, kNT);
    a = __uint_as_float(v << 16);
    b = __uint_as_float(v & 0xffff0000u);
}
__device__ __forceinline__ void row_load2(const float* row, int I, int i, float& a, float& b) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(row_rsrc(row, I * 4), i * 4, 0, kNT);
    a = __uint_as_float(v.x);
    b = __uint_as_float(v.y);
}
__device__ __forceinline__ void row_store2(float* row, int I, int i, float a, float b) {
    const u32x2 v = {__float_as_uint(a), __float_as_uint(b)};
    __builtin_amdgcn_raw_buffer_store_b64(v, row_rsrc(row, I * 4), i * 4, 0, kNT);
}
__device__ __forceinline__ float eval_span(const float4* t, int S, float xv, const GridK& g) {
    float u;
    const int s = span_u(xv, g, u);
    const bool in = (unsigned)s < (unsigned)S;
    const float4 a = t[in ? s : 0];
    const float v = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(a.w, u, a.z), u, a.y), u, a.x);
    return in ? v : 0.0f;
}

template <typename TS>
__global__ void __launch_bounds__(GP_T, 8) grouped_fwd2_kernel(GridK g, int N, int I, int groups, int R,
                                                               const TS* __restrict__ x,
                                                               const TS* __restrict__ C,
                                                               float* __restrict__ y) {
    extern __shared__ float4 tab[];
    const int S = g.G + 6;
    const int lane = threadIdx.x & (GP_C - 1), w = __builtin_amdgcn_readfirstlane(threadIdx.x / GP_C);
    const int i = blockIdx.x * GP_C2 + 2 * lane;
    const int c0 = blockIdx.x * GP_C2, c1 = min(c0 + GP_C2, I) - 1;
    BlockGroups bg;
    bg.g0 = group_of(c0, I, groups);
    bg.n = group_of(c1, I, groups) - bg.g0 + 1;
    build_table(tab, C, bg, g, false);
    __syncthreads();
    if (i >= I) return;                                // no barrier below
    const float4* t0 = tab + (group_of(i, I, groups) - bg.g0) * S;
    const float4* t1 = tab + (group_of(i + 1, I, groups) - bg.g0) * S;
    const int r0 = blockIdx.y * R, r1 = min(r0 + R, N);
    for (int b = r0 + w; b < r1; b += GP_W * GP_UF) {
        float xa[GP_UF], xb[GP_UF];
#pragma unroll
        for (int q = 0; q < GP_UF; ++q)
            row_load2(x + (int64_t)min(b + q * GP_W, r1 - 1) * I, I, i, xa[q], xb[q]);
#pragma unroll
        for (int q = 0; q < GP_UF; ++q) {
            const int row = b + q * GP_W;
            const float va = eval_span(t0, S, xa[q], g), vb = eval_span(t1, S, xb[q], g);
            row_store2(y + (int64_t)min(row, r1 - 1) * I, row < r1 ? I : 0, i, va, vb);
        }
    }
}

// Backward.  Same blocks as the forward.  LDS: acc [K+6][256] (thread t owns
// column t; row 3+m holds its sum for basis m), then the derivative table.
// At the end the 4 row waves' columns of a channel are added in wave order
// and written to the chunk's partials part[by][m][i].
template <typename TS, bool TAB>
__global__ void __launch_bounds__(GP_T, 4) grouped_bwd_kernel(GridK g, int N, int I, int groups, int R,
                                                              const TS* __restrict__ x,
                                                              const TS* __restrict__ C,
                                                              const float* __restrict__ dy,
                                                              float* __restrict__ dx,
                                                              float* __restrict__ part) {
    extern __shared__ float lds[];
    const int K = g.G + 3, S = g.G + 6;
    const int t = threadIdx.x, lane = t & (GP_C - 1), w = __builtin_amdgcn_readfirstlane(t / GP_C);
    const int i = blockIdx.x * GP_C + lane;
    const bool active = i < I;
    float* acc = lds;
    float4* tab = reinterpret_cast<float4*>(lds + (K + 6) * GP_T);
    const BlockGroups bg = block_groups(I, groups);
    if (TAB) build_table(tab, C, bg, g, true);
    if (part)
        for (int r = 0; r < K + 6; ++r) acc[r * GP_T + t] = 0.0f;
    __syncthreads();
    const int ic = active ? i : I - 1;
    const int gi = group_of(ic, I, groups);
    const float4* dt = tab + (gi - bg.g0) * S;
    const TS* c = C + (int64_t)gi * K;
    const int r0 = blockIdx.y * R, r1 = min(r0 + R, N);
    if (active) {
        for (int b = r0 + w; b < r1; b += GP_W * GP_UB) {
            float xv[GP_UB], dv[GP_UB];
#pragma unroll
            for (int q = 0; q < GP_UB; ++q) {
                const int64_t e = (int64_t)min(b + q * GP_W, r1 - 1) * I;
                xv[q] = load_at(x + e, i);
                dv[q] = load_at(dy + e, i);
            }
#pragma unroll
            for (int q = 0; q < GP_UB; ++q) {          // all rows computed, as in the forward
                const int row = b + q * GP_W;
                float u;
                const int s = span_u(xv[q], g, u);
                const bool in = (unsigned)s < (unsigned)S && row < r1;
                const int sc = in ? s : 0;
                const float d = in ? dv[q] : 0.0f;
                float deriv;
                if (TAB) {
                    const float4 a = dt[sc];
                    deriv = __builtin_fmaf(__builtin_fmaf(a.z, u, a.y), u, a.x);
                } else {
                    float p[4];
                    dpieces(u, g.scale, p[0], p[1], p[2], p[3]);
                    deriv = 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = sc - 3 + r;
                        if (m >= 0 && m < K) deriv = __builtin_fmaf(load_f(c, m), p[r], deriv);
                    }
                }
                if (dx && row < r1) __builtin_nontemporal_store(d * deriv, &at(dx + (int64_t)row * I, i));
                if (part) {
                    float p[4];
                    pieces(u, p[0], p[1], p[2], p[3]);
                    float* a = acc + sc * GP_T + t;    // rows sc .. sc+3 = basis sc-3 .. sc, padded by 3
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[r * GP_T] = __builtin_fmaf(d, p[r], a[r * GP_T]);
                }
            }
        }
    }
    if (!part) return;
    __syncthreads();
    for (int e = t; e < K * GP_C; e += GP_T) {
        const int m = e / GP_C, l = e - m * GP_C;
        const int ch = blockIdx.x * GP_C + l;
        if (ch >= I) continue;
        const float* a = acc + (m + 3) * GP_T + l;
        float v = a[0];
#pragma unroll
        for (int ww = 1; ww < GP_W; ++ww) v += a[ww * GP_C];
        part[((int64_t)blockIdx.y * K + m) * I + ch] = v;
    }
}

// red[m][i] = sum over the chunks q of part[q][m][i]: thread (l, r) of a block
// adds the chunks q = r, r+4, ... of column blockIdx.x*64 + l in order, then
// the 4 sums are added in r order.  With one group per channel the result is
// dC itself, written transposed (dC[i][m]).
__global__ void __launch_bounds__(256) grouped_sum_chunks_kernel(const float* __restrict__ part,
                                                                 float* __restrict__ red, int64_t KI,
                                                                 int64_t I, int K, int nq, int to_dC) {
    __shared__ float sh[4][64];
    const int l = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 64 + l;
    float v = 0.0f;
    if (e < KI) {
        int q = r;
        for (; q + 12 < nq; q += 16) {
            const float a0 = part[q * KI + e], a1 = part[(q + 4) * KI + e];
            const float a2 = part[(q + 8) * KI + e], a3 = part[(q + 12) * KI + e];
            v += a0;
            v += a1;
            v += a2;
            v += a3;
        }
        for (; q < nq; q += 4) v += part[q * KI + e];
    }
    sh[r][l] = v;
    __syncthreads();
    if (r == 0 && e < KI) {
        const float s = ((sh[0][l] + sh[1][l]) + sh[2][l]) + sh[3][l];
        if (to_dC) {
            const int64_t m = e / I, i = e - m * I;
            red[i * K + m] = s;
        } else {
            red[e] = s;
        }
    }
}

// dC[g, m] = sum over the group's channels i of red[m][i]: one wave per
// (g, m); lane l adds the channels ia + l, ia + l + 64, ... in order, then the
// lanes are added by a fixed butterfly.
__global__ void __launch_bounds__(256) grouped_sum_channels_kernel(const float* __restrict__ red,
                                                                   float* __restrict__ dC, int I,
                                                                   int groups, int K) {
    const int l = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= groups * K) return;                       // whole waves leave together
    const int gg = e / K, m = e - gg * K;
    // channels of group gg: the i with floor(i * groups / I) == gg
    const int ia = (int)(((int64_t)gg * I + groups - 1) / groups);
    const int ib = (int)(((int64_t)(gg + 1) * I + groups - 1) / groups);
    const float* rr = red + (int64_t)m * I;
    float v = 0.0f;
    for (int i = ia + l; i < ib; i += 64) v += rr[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (l == 0) dC[e] = v;
}

template <typename F>
hipError_t set_lds(F* kernel, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// the most groups that 64 consecutive channels meet
int64_t max_block_groups(int64_t I, int groups) {
    return std::min<int64_t>(std::min<int64_t>(GP_C, I), groups);
}

size_t table_bytes(int64_t I, int groups, int G) { return (size_t)max_block_groups(I, groups) * (G + 6) * 16; }

template <typename TS, bool TAB>
hipError_t fwd_t(const GridK& g, const GroupPlan& gp, int64_t N, int64_t I, int groups, const void* x,
                 const void* C, float* y, hipStream_t s) {
    const size_t lds = TAB ? table_bytes(I, groups, g.G) : 0;
    hipError_t e = set_lds(grouped_fwd_kernel<TS, TAB>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_fwd_kernel<TS, TAB>), dim3((unsigned)gp.xb, (unsigned)gp.gy_fwd), dim3(GP_T),
                       lds, s, g, (int)N, (int)I, groups, (int)gp.rows_fwd, static_cast<const TS*>(x),
                       static_cast<const TS*>(C), y);
    return hipGetLastError();
}

template <typename TS, bool TAB>
hipError_t bwd_t(const GridK& g, const GroupPlan& gp, int64_t N, int64_t I, int groups, const void* x,
                 const void* C, const float* dy, float* dx, float* part, hipStream_t s) {
    const size_t lds = (size_t)(g.G + 9) * GP_T * 4 + (TAB ? table_bytes(I, groups, g.G) : 0);
    hipError_t e = set_lds(grouped_bwd_kernel<TS, TAB>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_bwd_kernel<TS, TAB>), dim3((unsigned)gp.xb, (unsigned)gp.gy_bwd), dim3(GP_T),
                       lds, s, g, (int)N, (int)I, groups, (int)gp.rows_bwd, static_cast<const TS*>(x),
                       static_cast<const TS*>(C), dy, dx, part);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_fwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, float* y, hipStream_t s) {
    if (N == 0) return hipSuccess;
    const size_t tab2 = (size_t)std::min<int64_t>(std::min<int64_t>(GP_C2, I), groups) * (g.G + 6) * 16;
    if (I % 2 == 0 && tab2 <= kTabLimit) {
        const int64_t xb2 = (I + GP_C2 - 1) / GP_C2;
        const int64_t gy0 = std::max<int64_t>(1, 2048 / xb2);
        const int64_t rows = round_up((N + gy0 - 1) / gy0, GP_W * GP_UF);
        const int64_t gy = (N + rows - 1) / rows;
        hipError_t e = dtype == KAN_F32 ? set_lds(grouped_fwd2_kernel<float>, tab2)
                                        : set_lds(grouped_fwd2_kernel<uint16_t>, tab2);
        if (e != hipSuccess) return e;
        if (dtype == KAN_F32)
            hipLaunchKernelGGL(grouped_fwd2_kernel<float>, dim3((unsigned)xb2, (unsigned)gy), dim3(GP_T), tab2, s, g,
                               (int)N, (int)I, groups, (int)rows, static_cast<const float*>(x),
                               static_cast<const float*>(C), y);
        else
            hipLaunchKernelGGL(grouped_fwd2_kernel<uint16_t>, dim3((unsigned)xb2, (unsigned)gy), dim3(GP_T), tab2, s,
                               g, (int)N, (int)I, groups, (int)rows, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(C), y);
        return hipGetLastError();
    }
    const GroupPlan gp = grouped_plan(N, I, g.G + 3);
    const bool tab = table_bytes(I, groups, g.G) <= kTabLimit;
    if (dtype == KAN_F32)
        return tab ? fwd_t<float, true>(g, gp, N, I, groups, x, C, y, s)
                   : fwd_t<float, false>(g, gp, N, I, groups, x, C, y, s);
    return tab ? fwd_t<uint16_t, true>(g, gp, N, I, groups, x, C, y, s)
               : fwd_t<uint16_t, false>(g, gp, N, I, groups, x, C, y, s);
}

hipError_t launch_grouped_bwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, const float* dy, float* dx, float* dC,
                              float* part, float* red, hipStream_t s) {
    const int K = g.G + 3;
    if (N == 0) return dC ? launch_fill_zero(dC, (int64_t)groups * K, s) : hipSuccess;
    const GroupPlan gp = grouped_plan(N, I, K);
    const bool tab = table_bytes(I, groups, g.G) <= kTabLimit;
    float* p = dC ? part : nullptr;
    hipError_t e;
    if (dtype == KAN_F32)
        e = tab ? bwd_t<float, true>(g, gp, N, I, groups, x, C, dy, dx, p, s)
                : bwd_t<float, false>(g, gp, N, I, groups, x, C, dy, dx, p, s);
    else
        e = tab ? bwd_t<uint16_t, true>(g, gp, N, I, groups, x, C, dy, dx, p, s)
                : bwd_t<uint16_t, false>(g, gp, N, I, groups, x, C, dy, dx, p, s);
    if (e != hipSuccess || !dC) return e;
    const int64_t KI = (int64_t)K * I;
    const int per_channel = groups == I;
    hipLaunchKernelGGL(grouped_sum_chunks_kernel, dim3((unsigned)((KI + 63) / 64)), dim3(256), 0, s, part,
                       per_channel ? dC : red, KI, I, K, (int)gp.gy_bwd, per_channel);
    if ((e = hipGetLastError()) != hipSuccess || per_channel) return e;
    hipLaunchKernelGGL(grouped_sum_channels_kernel, dim3((unsigned)(((int64_t)groups * K + 3) / 4)), dim3(256),
                       0, s, red, dC, (int)I, groups, K);
    return hipGetLastError();
}

}  // namespace kan
