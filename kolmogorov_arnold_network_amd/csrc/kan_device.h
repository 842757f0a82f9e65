// Device-side pieces shared by every kernel of the KAN layer library (gfx950).
//
// Knot span and local coordinate, the 4 non-zero cubic pieces and their
// derivatives, and the silu base branch.  The pages' recommendation (InKAN
// project page, "Why InKAN?"): evaluate the stable piecewise polynomials of the
// one knot span that holds x instead of running the Cox-de Boor recursion, and
// touch only the 4 basis functions that are non-zero there.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kan {

// Grid constants derived once on the host.  v = x * scale + shift is the
// position of x in knot units measured from the first knot t_0 = lo - 3h.
struct GridK {
    float scale;  // G / (hi - lo) = 1 / h
    float shift;  // 3 - lo * G / (hi - lo)
    int G;        // intervals; basis functions m = 0 .. G+2
};

// Span index s (t_s <= x < t_{s+1}) and local coordinate u in [0, 1].
// u is produced by one fused multiply-add against the integer s, so it is
// rounded once; a naive (x - t_s) / h loses up to 2^-19 at G = 50.  The
// rounded position v can land on the next integer when x sits just below a
// knot; the residual is then negative and the span steps back by one.
// Non-finite x yields an out-of-range span (no basis function is touched).
__device__ __forceinline__ int span_u(float x, const GridK& g, float& u) {
    float v = __builtin_fmaf(x, g.scale, g.shift);
    v = __builtin_fminf(__builtin_fmaxf(v, -8.0f), 16777216.0f);  // NaN -> -8
    float fs = __builtin_floorf(v);
    if (__builtin_fmaf(x, g.scale, g.shift - fs) < 0.0f) fs -= 1.0f;
    const float w = __builtin_fmaf(x, g.scale, g.shift - fs);
    u = __builtin_fminf(__builtin_fmaxf(w, 0.0f), 1.0f);
    return (int)fs;
}

// Uniform cubic B-spline pieces on a span, by local coordinate u: the basis
// functions m = s-3 .. s take b0 .. b3.  Written so that every term is
// non-negative (InKAN page, "Why InKAN?": guaranteed non-negative output, no
// alternating sums): b1 = (4 - 6u^2 + 3u^3)/6 >= 1/6 on [0, 1], b2 the same
// in w = 1 - u.
__device__ __forceinline__ void pieces(float u, float& b0, float& b1, float& b2, float& b3) {
    const float w = 1.0f - u;
    const float u2 = u * u, w2 = w * w;
    const float s6 = 1.0f / 6.0f;
    b0 = w2 * w * s6;
    b3 = u2 * u * s6;
    b1 = __builtin_fmaf(u2, __builtin_fmaf(3.0f, u, -6.0f), 4.0f) * s6;
    b2 = __builtin_fmaf(w2, __builtin_fmaf(3.0f, w, -6.0f), 4.0f) * s6;
}

// The same pieces with the 1/6 folded into the coefficients, two multiplies
// fewer: b1 = u^2 (u/2 - 1) + 2/3 >= 1/6 on [0, 1] (b2 the same in w).  Its
// rounding differs from pieces() by about an ulp, which a bf16 tile never
// sees; the float32 paths keep pieces().
__device__ __forceinline__ void pieces_fast(float u, float& b0, float& b1, float& b2, float& b3) {
    const float w = 1.0f - u;
    const float u2 = u * u, w2 = w * w;
    const float s6 = 1.0f / 6.0f, t3 = 2.0f / 3.0f;
    b0 = w2 * (w * s6);
    b3 = u2 * (u * s6);
    b1 = __builtin_fmaf(u2, __builtin_fmaf(0.5f, u, -1.0f), t3);
    b2 = __builtin_fmaf(w2, __builtin_fmaf(0.5f, w, -1.0f), t3);
}

// Truncated-power form of one basis function (FlashKAN project page: five
// shifted (x)_+^3 terms with the normalised coordinate clamped to [0, k+1]):
// u = (x - t_m) / h clamped to [0, 4], and
//   B_m = (u^3 - 4 (u-1)_+^3 + 6 (u-2)_+^3 - 4 (u-3)_+^3) / 6
//   B'_m = (u^2 - 4 (u-1)_+^2 + 6 (u-2)_+^2 - 4 (u-3)_+^2) / 2 * (1/h),
// the fifth term (u-4)_+ being 0 under the clamp.  Needs no span, but the
// alternating sum cancels: near u = 4 terms of size 64 leave a result near 0,
// so float32 loses up to ~1e-5 and may round below 0.
__device__ __forceinline__ void tp_basis(float u, float scale, float& b, float& d) {
    u = __builtin_fminf(__builtin_fmaxf(u, 0.0f), 4.0f);
    const float p1 = __builtin_fmaxf(u - 1.0f, 0.0f), p2 = __builtin_fmaxf(u - 2.0f, 0.0f),
                p3 = __builtin_fmaxf(u - 3.0f, 0.0f);
    const float q0 = u * u, q1 = p1 * p1, q2 = p2 * p2, q3 = p3 * p3;
    b = (q0 * u - 4.0f * (q1 * p1) + 6.0f * (q2 * p2) - 4.0f * (q3 * p3)) * (1.0f / 6.0f);
    d = (q0 - 4.0f * q1 + 6.0f * q2 - 4.0f * q3) * (0.5f * scale);
}

// d/dx of the same pieces: (db/du) * (du/dx), du/dx = 1/h = scale.
__device__ __forceinline__ void dpieces(float u, float scale, float& d0, float& d1, float& d2,
                                        float& d3) {
    const float w = 1.0f - u;
    const float hs = 0.5f * scale;
    d0 = -(w * w) * hs;
    d1 = u * __builtin_fmaf(3.0f, u, -4.0f) * hs;
    d2 = -(w * __builtin_fmaf(3.0f, w, -4.0f)) * hs;
    d3 = (u * u) * hs;
}

// The D + 1 non-zero uniform B-splines of degree D (1 <= D <= 5, a runtime
// value uniform across the wave) on a knot span with local coordinate u, and
// their x-derivatives: value r belongs to basis function s - D + r.  The
// degree-by-degree recurrence on uniform knots,
//     N^q_r = ((u + q - r) N^{q-1}_{r-1} + (r + 1 - u) N^{q-1}_r) / q,
// adds non-negative terms only on [0, 1]; dN^D_r/dx = (N^{D-1}_{r-1} -
// N^{D-1}_r) / h.  Entries r > D are zero.
__device__ __forceinline__ void local_basis_rt(float u, float scale, int D, float b[6], float d[6]) {
    float N[6] = {1.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 6; ++r) d[r] = 0.0f;
#pragma unroll
    for (int q = 1; q <= 5; ++q) {
        if (q > D) break;
        if (q == D) {
#pragma unroll
            for (int r = 0; r < 6; ++r)
                if (r <= q) d[r] = ((r >= 1 ? N[r - 1] : 0.0f) - (r <= q - 1 ? N[r] : 0.0f)) * scale;
        }
        const float inv = 1.0f / (float)q;
#pragma unroll
        for (int r = 5; r >= 0; --r) {
            if (r > q) continue;
            float v = r >= 1 ? (u + (float)(q - r)) * N[r - 1] : 0.0f;
            if (r <= q - 1) v = __builtin_fmaf((float)(r + 1) - u, N[r], v);
            N[r] = v * inv;
        }
    }
#pragma unroll
    for (int r = 0; r < 6; ++r) b[r] = N[r];
}

// silu(x) = x * sigmoid(x) and its derivative sigmoid(x) * (1 + x (1 - sigmoid(x))).
__device__ __forceinline__ float silu(float x) {
    const float e = __expf(-x);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float silu_prime(float x) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-x));
    return s * __builtin_fmaf(x, 1.0f - s, 1.0f);
}

// Storage types.
__device__ __forceinline__ float load_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_f(const uint16_t* p, int64_t i) {
    return __uint_as_float(((uint32_t)p[i]) << 16);
}
// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace kan
