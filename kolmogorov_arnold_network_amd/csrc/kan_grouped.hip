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
// and written once, so the kernels stream HBM.  dC is reduced without atomics:
// a block owns 256 channels and a contiguous chunk of rows, every thread adds
// its channel's terms into a private LDS column in row order, and two
// fixed-order passes add the per-block partials over the chunks and then over
// the channels of each group.
#include "kan_internal.h"

namespace kan {

namespace {

constexpr int GP_T = 256;    // channels per block, one per thread
constexpr int GP_U = 4;      // rows whose loads are issued together

__device__ __forceinline__ int group_of(int i, int I, int groups) {
    return (int)(((int64_t)i * groups) / I);
}

// Coefficients the block's threads read: staged in LDS (STAGE) as the rows of
// the groups g0 .. g1 that its channels meet, else read from memory.
template <typename TS, bool STAGE>
struct Coef {
    const float* lds;
    const TS* mem;
    __device__ __forceinline__ float operator()(int m) const {
        if constexpr (STAGE) return lds[m];
        else return load_f(mem, m);
    }
};

template <typename TS, bool STAGE>
__device__ __forceinline__ Coef<TS, STAGE> block_coef(float* cs, const TS* C, int K, int I, int groups) {
    const int i0 = blockIdx.x * GP_T;
    const int i = min(i0 + (int)threadIdx.x, I - 1);
    Coef<TS, STAGE> c;
    c.mem = C + (int64_t)group_of(i, I, groups) * K;
    c.lds = cs;
    if constexpr (STAGE) {
        const int g0 = group_of(i0, I, groups), g1 = group_of(min(i0 + GP_T, I) - 1, I, groups);
        for (int e = threadIdx.x; e < (g1 - g0 + 1) * K; e += GP_T) cs[e] = load_f(C, (int64_t)g0 * K + e);
        __syncthreads();
        c.lds = cs + (group_of(i, I, groups) - g0) * K;
    }
    return c;
}

// Forward.  Block (bx, by): channels bx*256 .. +255, rows by*R .. by*R+R-1.
template <typename TS, bool STAGE>
__global__ void __launch_bounds__(GP_T) grouped_fwd_kernel(GridK g, int N, int I, int groups, int R,
                                                           const TS* __restrict__ x,
                                                           const TS* __restrict__ C,
                                                           float* __restrict__ y) {
    extern __shared__ float cs[];
    const int K = g.G + 3;
    const Coef<TS, STAGE> c = block_coef<TS, STAGE>(cs, C, K, I, groups);
    const int i = blockIdx.x * GP_T + threadIdx.x;
    if (i >= I) return;                                // no barrier below
    const int r0 = blockIdx.y * R, r1 = min(r0 + R, N);
    for (int b = r0; b < r1; b += GP_U) {
        float xv[GP_U];
#pragma unroll
        for (int q = 0; q < GP_U; ++q) xv[q] = load_f(x, (int64_t)min(b + q, r1 - 1) * I + i);
#pragma unroll
        for (int q = 0; q < GP_U; ++q) {
            if (b + q >= r1) break;
            float u, w[4];
            const int s = span_u(xv[q], g, u);
            pieces(u, w[0], w[1], w[2], w[3]);
            float v = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = s - 3 + r;
                if (m >= 0 && m < K) v = __builtin_fmaf(c(m), w[r], v);
            }
            y[(int64_t)(b + q) * I + i] = v;
        }
    }
}

// Backward.  Same blocks as the forward; thread i writes dx[b, i] and adds
// dy[b, i] * B_m(x[b, i]) into its own LDS column acc[m][t] in row order,
// then writes the column to the partials part[by][m][i].
template <typename TS, bool STAGE>
__global__ void __launch_bounds__(GP_T) grouped_bwd_kernel(GridK g, int N, int I, int groups, int R,
                                                           const TS* __restrict__ x,
                                                           const TS* __restrict__ C,
                                                           const float* __restrict__ dy,
                                                           float* __restrict__ dx,
                                                           float* __restrict__ part) {
    extern __shared__ float lds[];                     // acc [K][256], then the staged coefficients
    const int K = g.G + 3;
    const int t = threadIdx.x;
    float* acc = lds;
    const Coef<TS, STAGE> c = block_coef<TS, STAGE>(lds + K * GP_T, C, K, I, groups);
    const int i = blockIdx.x * GP_T + t;
    if (i >= I) return;                                // no barrier below: columns are private
    if (part)
        for (int m = 0; m < K; ++m) acc[m * GP_T + t] = 0.0f;
    const int r0 = blockIdx.y * R, r1 = min(r0 + R, N);
    for (int b = r0; b < r1; b += GP_U) {
        float xv[GP_U], dv[GP_U];
#pragma unroll
        for (int q = 0; q < GP_U; ++q) {
            const int64_t e = (int64_t)min(b + q, r1 - 1) * I + i;
            xv[q] = load_f(x, e);
            dv[q] = dy[e];
        }
#pragma unroll
        for (int q = 0; q < GP_U; ++q) {
            if (b + q >= r1) break;
            float u, w[4], dw[4];
            const int s = span_u(xv[q], g, u);
            dpieces(u, g.scale, dw[0], dw[1], dw[2], dw[3]);
            float v = 0.0f;
            if (part) pieces(u, w[0], w[1], w[2], w[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = s - 3 + r;
                if (m >= 0 && m < K) {
                    v = __builtin_fmaf(c(m), dw[r], v);
                    if (part) acc[m * GP_T + t] = __builtin_fmaf(dv[q], w[r], acc[m * GP_T + t]);
                }
            }
            if (dx) dx[(int64_t)(b + q) * I + i] = dv[q] * v;
        }
    }
    if (part)
        for (int m = 0; m < K; ++m) part[((int64_t)blockIdx.y * K + m) * I + i] = acc[m * GP_T + t];
}

// red[m][i] = sum over chunks by = 0 .. nby-1, in that order, of part[by][m][i]
__global__ void grouped_sum_rows_kernel(const float* __restrict__ part, float* __restrict__ red,
                                        int64_t KI, int nby) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < KI;
         e += (int64_t)gridDim.x * blockDim.x) {
        float v = 0.0f;
        for (int q = 0; q < nby; ++q) v += part[q * KI + e];
        red[e] = v;
    }
}

// dC[g, m] = sum over the group's channels i, in order, of red[m][i]
__global__ void grouped_sum_channels_kernel(const float* __restrict__ red, float* __restrict__ dC,
                                            int I, int groups, int K) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= groups * K) return;
    const int gg = e / K, m = e - gg * K;
    // channels of group gg: the i with floor(i * groups / I) == gg
    const int ia = (int)(((int64_t)gg * I + groups - 1) / groups);
    const int ib = (int)(((int64_t)(gg + 1) * I + groups - 1) / groups);
    float v = 0.0f;
    for (int i = ia; i < ib; ++i) v += red[(int64_t)m * I + i];
    dC[e] = v;
}

// LDS bytes of the coefficient rows a block meets (at most one group per channel)
size_t coef_lds(int64_t I, int groups, int K) {
    return (size_t)std::min<int64_t>(std::min<int64_t>(GP_T, I), groups) * K * 4;
}
constexpr size_t kStageLimit = 32 * 1024;

template <typename F>
hipError_t set_lds(F* kernel, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename TS, bool STAGE>
hipError_t fwd_t(const GridK& g, const GroupPlan& gp, int64_t N, int64_t I, int groups, const void* x,
                 const void* C, float* y, hipStream_t s) {
    const size_t lds = STAGE ? coef_lds(I, groups, g.G + 3) : 0;
    hipError_t e = set_lds(grouped_fwd_kernel<TS, STAGE>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_fwd_kernel<TS, STAGE>), dim3((unsigned)gp.xb, (unsigned)gp.gy_fwd),
                       dim3(GP_T), lds, s, g, (int)N, (int)I, groups, (int)gp.rows_fwd,
                       static_cast<const TS*>(x), static_cast<const TS*>(C), y);
    return hipGetLastError();
}

template <typename TS, bool STAGE>
hipError_t bwd_t(const GridK& g, const GroupPlan& gp, int64_t N, int64_t I, int groups, const void* x,
                 const void* C, const float* dy, float* dx, float* part, hipStream_t s) {
    const int K = g.G + 3;
    const size_t lds = (size_t)K * GP_T * 4 + (STAGE ? coef_lds(I, groups, K) : 0);
    hipError_t e = set_lds(grouped_bwd_kernel<TS, STAGE>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_bwd_kernel<TS, STAGE>), dim3((unsigned)gp.xb, (unsigned)gp.gy_bwd),
                       dim3(GP_T), lds, s, g, (int)N, (int)I, groups, (int)gp.rows_bwd,
                       static_cast<const TS*>(x), static_cast<const TS*>(C), dy, dx, part);
    return hipGetLastError();
}

}  // namespace

// Row chunks.  The forward aims at 2048 blocks (8 per CU).  The backward aims
// at 1024 and gives every chunk at least max(64, 24 K) rows, so that the
// partials (K floats per channel per chunk, written and read back) stay
// within about 1/30 of the traffic of x, dy and dx.
GroupPlan grouped_plan(int64_t N, int64_t I, int K) {
    GroupPlan gp;
    gp.xb = (I + GP_T - 1) / GP_T;
    auto chunk = [&](int64_t blocks, int64_t rmin) {
        const int64_t gy = std::max<int64_t>(1, (blocks + gp.xb - 1) / gp.xb);
        return round_up(std::max<int64_t>(rmin, (N + gy - 1) / gy), GP_U);
    };
    gp.rows_fwd = chunk(2048, 16);
    gp.rows_bwd = chunk(1024, std::max<int64_t>(64, 24 * (int64_t)K));
    gp.gy_fwd = (N + gp.rows_fwd - 1) / gp.rows_fwd;
    gp.gy_bwd = (N + gp.rows_bwd - 1) / gp.rows_bwd;
    gp.part_floats = gp.gy_bwd * K * I;
    gp.red_floats = (int64_t)K * I;
    return gp;
}

hipError_t launch_grouped_fwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, float* y, hipStream_t s) {
    if (N == 0) return hipSuccess;
    const GroupPlan gp = grouped_plan(N, I, g.G + 3);
    const bool stage = coef_lds(I, groups, g.G + 3) <= kStageLimit;
    if (dtype == KAN_F32)
        return stage ? fwd_t<float, true>(g, gp, N, I, groups, x, C, y, s)
                     : fwd_t<float, false>(g, gp, N, I, groups, x, C, y, s);
    return stage ? fwd_t<uint16_t, true>(g, gp, N, I, groups, x, C, y, s)
                 : fwd_t<uint16_t, false>(g, gp, N, I, groups, x, C, y, s);
}

hipError_t launch_grouped_bwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, const float* dy, float* dx, float* dC,
                              float* part, float* red, hipStream_t s) {
    const int K = g.G + 3;
    if (N == 0) return dC ? launch_fill_zero(dC, (int64_t)groups * K, s) : hipSuccess;
    const GroupPlan gp = grouped_plan(N, I, K);
    const bool stage = coef_lds(I, groups, K) <= kStageLimit;
    float* p = dC ? part : nullptr;
    hipError_t e;
    if (dtype == KAN_F32)
        e = stage ? bwd_t<float, true>(g, gp, N, I, groups, x, C, dy, dx, p, s)
                  : bwd_t<float, false>(g, gp, N, I, groups, x, C, dy, dx, p, s);
    else
        e = stage ? bwd_t<uint16_t, true>(g, gp, N, I, groups, x, C, dy, dx, p, s)
                  : bwd_t<uint16_t, false>(g, gp, N, I, groups, x, C, dy, dx, p, s);
    if (e != hipSuccess || !dC) return e;
    const int64_t KI = (int64_t)K * I;
    hipLaunchKernelGGL(grouped_sum_rows_kernel, dim3((unsigned)std::min<int64_t>((KI + 255) / 256, 16384)),
                       dim3(256), 0, s, part, red, KI, (int)gp.gy_bwd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(grouped_sum_channels_kernel, dim3((unsigned)((groups * K + 255) / 256)), dim3(256), 0,
                       s, red, dC, (int)I, groups, K);
    return hipGetLastError();
}

}  // namespace kan
