// Host-side plan of one KAN layer call and the kernel launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "kan.h"
#include "kan_device.h"

namespace kan {

// MFMA tile geometry (both dtypes): 256 x 256 output tile per workgroup of
// 8 waves (4 x 2, 64 x 128 each), k-tiles of 128 bytes per row (64 bf16 or
// 32 float) staged in LDS with a 144-byte row pitch, two stages.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileKBytes = 128;

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

struct Plan {
    int64_t N, I, O;
    int G, K, Kb;        // K = G+3 spline functions; Kb = K + has_base columns per input
    int base;
    int dtype;           // KAN_F32 / KAN_BF16
    // 2-D tensor-product layer: "inputs" are the P pairs (x[b, 2p], x[b, 2p+1]),
    // K = Kb = (G+3)^2 columns per pair (m for the first input, n for the
    // second, n fastest); x rows are xI = 2P wide.  One-dimensional: pair = 0,
    // xI = I.
    int pair;
    int64_t xI;
    int degree;          // spline degree, 1 .. 5 (the gather kernels, the sparse
                         // forward and the 2-D layer are cubic only)
    int variant_fwd;     // resolved per pass: KAN_VARIANT_MFMA or KAN_VARIANT_GATHER
    int variant_bwd;
    int esize;           // bytes per stored element (4 or 2)
    GridK gk;

    // MFMA geometry
    int BK;              // elements per k-tile (128 bytes)
    int64_t IKb;         // I * Kb: width of the dense basis
    int64_t Opad;        // O rounded up to the tile (rows of the packed C')
    int64_t Npad;        // N rounded up to the tile
    int64_t Kf;          // forward contraction length: IKb rounded up to BK
    int64_t tiles_dx;    // n-tiles of the dx contraction: ceil(I * Kb / 256)

    // structured-sparse forward (bf16): each input's Kb columns become NG
    // groups of 4 (Kb8 = 4 NG columns) in the column order of kan_sparse.h
    int sparse;          // 1: the forward uses the sparse layout
    int NG, Kb8;
    int64_t Kfs;         // sparse forward contraction length: I * Kb8 rounded up to 64

    // k-split of launches with too few output tiles: the forward (over its
    // k-tiles) and dC (over the batch) run as split_* slices of nks_* k-tiles
    // that write fp32 partial outputs, summed afterwards in slice order
    int split_fwd, split_dc;
    int64_t nks_fwd, nks_dc;

    // workspace layout (bytes); forward uses [off_cp, +sz_cp).  Every array is
    // blocked: 256-row tiles, each cut into k-tiles of 256 x BK contiguous
    // elements.
    size_t off_cp, sz_cp;      // C': rows j < Opad, k = (i, m) < Kf (sparse: < Kfs, permuted)
    size_t off_cpt, sz_cpt;    // C'^T: tiles_dx tiles of 256 consecutive columns of C', k = j < Opad
    size_t off_dyp, sz_dyp;    // dy in storage dtype: rows b < Npad, k = j < Opad
    size_t off_dyt, sz_dyt;    // dy^T in storage dtype: rows j < Opad, k = b < Npad
    size_t off_part, sz_part;  // dx partial sums of inputs cut by a tile edge: [Npad][tiles_dx][2] float
                               // (pairs: [Npad][tiles_dx][2][2], both inputs of the pair)
    size_t off_yp, sz_yp;      // forward slices' partial y: [split_fwd][N][O] float (split_fwd > 1)
    size_t off_dcp, sz_dcp;    // dC slices' partials: [split_dc][O][I][K] then [split_dc][O][I] float
    size_t ws_fwd, ws_bwd;
};

// Builds the plan; returns KAN_OK or the validation error for `desc` alone.
int make_plan(const kan_desc_t* desc, Plan* p);
// The plan of a 2-D tensor-product layer (always on the matrix cores).
int make_plan_surface(const kan_surface_desc_t* desc, Plan* p);

// ---- launchers (return hipError_t of the launch) ----
// degree 1 .. 5; g built for that degree (t_0 = lo - degree h)
hipError_t launch_basis_eval(const GridK& g, int64_t n, int dtype, const void* x, float* B,
                             float* dB, bool truncated_power, int degree, hipStream_t s);
hipError_t launch_cast_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

hipError_t launch_gather_fwd(const Plan& p, const void* x, const void* C, const void* W,
                             float* y, hipStream_t s);
hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void* W,
                            const float* dy, float* dx, hipStream_t s);
hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                            hipStream_t s);

hipError_t launch_pack_fwd(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s);
hipError_t launch_pack_fwd_sparse(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s);
hipError_t launch_pack_bwd(const Plan& p, const void* C, const void* W, void* cpt, hipStream_t s);
hipError_t launch_prep_dy(const Plan& p, const float* dy, void* dyp, void* dyt, hipStream_t s);
hipError_t launch_mfma_fwd(const Plan& p, const void* x, const void* cp, float* ypart, float* y,
                           hipStream_t s);
hipError_t launch_mfma_dx(const Plan& p, const void* x, const void* dyp, const void* cpt,
                          float* part, float* dx, hipStream_t s);
hipError_t launch_mfma_dc(const Plan& p, const void* x, const void* dyt, float* cpart, float* dC,
                          float* dW, hipStream_t s);

// Grouped spline activation: blocks of 256 channels by chunks of rows.
struct GroupPlan {
    int64_t xb;                  // channel blocks: ceil(I / 256)
    int64_t rows_fwd, gy_fwd;    // forward: rows per chunk, chunks
    int64_t rows_bwd, gy_bwd;    // backward: rows per chunk, chunks (= partial sets of dC)
    int64_t part_floats;         // gy_bwd * K * I: per-chunk partials of the per-channel dC
    int64_t red_floats;          // K * I: partials summed over the chunks
};
GroupPlan grouped_plan(int64_t N, int64_t I, int K);
hipError_t launch_grouped_fwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, float* y, hipStream_t s);
hipError_t launch_grouped_bwd(const GridK& g, int64_t N, int64_t I, int groups, int dtype,
                              const void* x, const void* C, const float* dy, float* dx, float* dC,
                              float* part, float* red, hipStream_t s);

}  // namespace kan
