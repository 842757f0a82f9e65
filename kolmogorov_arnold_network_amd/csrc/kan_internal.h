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

// Block geometry of the vector-ALU kernels, shared with their host plans
// (kan_plan.cpp).
constexpr int kGatherFwdOutputs = 64;   // local-gather forward: outputs per block
constexpr int kGatherDxRows = 256;      // local-gather dx: rows per block
constexpr int kGatherDxInputs = 16;     // local-gather dx: inputs per block
constexpr int kGatherDcRecord = 8;      // local-gather dC: floats of a row's weight record
constexpr int kGroupChannels = 64;      // grouped activation: channels per block (one per lane)
constexpr int kGroupWaves = 4;          // grouped activation: row waves per block
constexpr int kGroupRowsFwd = 16;       // grouped forward: rows whose loads a thread issues together
constexpr int kGroupRowsBwd = 8;        // grouped backward: the same

// Local-gather forward: blocks of nt threads compute nt / 4 rows by 64
// outputs, staging ic inputs per chunk in lds bytes of LDS; the inputs are
// cut into `split` slices of `is` inputs (split > 1: float64 partial outputs
// [split][N][O] in a workspace of ws bytes, added in slice order).
struct GatherFwdPlan {
    int nt, ic, split;
    int64_t is, rb, ob;
    size_t lds, ws;
};
GatherFwdPlan gather_fwd_plan(int64_t N, int64_t I, int64_t O, int K, int D, int base);

// Local-gather backward.  dx: blocks of 1024 threads compute 256 rows by 16
// inputs (rb x ib blocks), summing over outputs in chunks of jc staged in
// lds_dx bytes; the outputs are cut into sx slices of js (sx > 1: float32
// partial dx [sx][N][I] at off_dxp).  dC: blocks of nt_dc threads, one input
// per wave and 64 opl outputs (ibn x ob blocks), kmax register sums per output,
// lds_dc bytes; the rows are cut into sc slices of rs (sc > 1: partial dC
// [sc][O][I][K] at off_dcp and dW_base [sc][O][I] at off_dwp).
struct GatherBwdPlan {
    int jc, sx, kmax, opl, nt_dc, sc;
    int64_t rb, ib, js, ibn, ob, rs;
    size_t lds_dx, lds_dc, off_dxp, off_dcp, off_dwp, ws;
};
GatherBwdPlan gather_bwd_plan(int64_t N, int64_t I, int64_t O, int K, int base);

struct GatherDxArgs {
    GridK g;
    int N, I, O, base;
    int RB, IB;          // row blocks, input blocks
    int JS;              // outputs per slice (a multiple of the chunk)
    float invK;          // 1 / K, rounded
    const void* x;
    const void* C;
    const void* W;
    const float* dy;
    float* dx;           // one slice: the output
    float* part;         // several slices: their partial dx [slice][N][I]
};

struct GatherDcArgs {
    GridK g;
    int N, I, O;
    int IBN, OB;         // input blocks, output blocks
    int RS;              // rows per slice (a multiple of 64)
    int bf16;            // x stored as bf16
    const void* x;
    const float* dy;
    float* dC;           // one slice: the outputs (either may be NULL)
    float* dW;
    float* cpart;        // several slices: partial dC [slice][O][I][K]
    float* wpart;        // and dW_base [slice][O][I]
};

struct GatherFwdArgs {
    GridK g;
    int N, I, O;
    int IC, IS;          // inputs per chunk and per slice
    int RB, OB;          // row blocks and output blocks of one slice
    const void* x;
    const void* C;
    const void* W;
    float* y;            // one slice: the output
    double* part;        // several slices: their partial outputs [slice][N][O]
};

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
    int degree;          // spline degree, 1 .. 5 (the sparse forward and the 2-D
                         // layer are cubic only)
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
    int tp;              // 1: the dense bf16 forward generates its basis by the
                         // truncated-power form (KAN_FLAG_TP_FORWARD)
    int sparse;          // 1: the forward uses the sparse layout
    int NG, Kb8;
    int64_t Kfs;         // sparse forward contraction length: I * Kb8 rounded up to 64

    // k-split of launches whose output tiles leave CUs idle: the forward
    // (over its k-tiles) and dC (over the batch).  The last tail_* tile rows
    // (every row, or the few that would run in a final, mostly idle round)
    // run as split_* slices of nks_* k-tiles that write fp32 partial outputs,
    // summed afterwards in slice order; the other tile rows run whole and
    // write their outputs directly.
    int split_fwd, split_dc;
    int64_t nks_fwd, nks_dc;
    int64_t tail_fwd, tail_dc;

    // workspace layout (bytes); forward uses [off_cp, +sz_cp).  Every array is
    // blocked: 256-row tiles, each cut into k-tiles of 256 x BK contiguous
    // elements.
    size_t off_cp, sz_cp;      // C': rows j < Opad, k = (i, m) < Kf (sparse: < Kfs, permuted)
    size_t off_cpt, sz_cpt;    // C'^T: tiles_dx tiles of 256 consecutive columns of C', k = j < Opad
    size_t off_dyp, sz_dyp;    // dy in storage dtype: rows b < Npad, k = j < Opad
    size_t off_dyt, sz_dyt;    // dy^T in storage dtype: rows j < Opad, k = b < Npad
    size_t off_part, sz_part;  // dx partial sums of inputs cut by a tile edge: [Npad][tiles_dx][2] float
                               // (pairs: [Npad][tiles_dx][2][2], both inputs of the pair)
    // basis operands built once in HBM (bf16 cubic layers with Kb <= 12 and
    // at least 8 (forward) or 3 (dC) output tiles): the forward's A operand
    // Phi' [Npad][Kf] and dC's B operand Phi'^T [tiles_dx * 256][Npad],
    // blocked like the others
    int mat_fwd, mat_dc;
    size_t off_phi, sz_phi;    // forward workspace
    size_t off_phit, sz_phit;  // backward workspace
    size_t off_yp, sz_yp;      // forward slices' partial y of the tail rows: [split_fwd][fwd_tail_rows][O] float
    size_t off_dcp, sz_dcp;    // dC slices' partials of the tail rows j: [split_dc][dc_tail_rows][I][K], then
                               // [split_dc][dc_tail_rows][I] float
    size_t ws_fwd, ws_bwd;

    GatherFwdPlan gf;    // the local-gather forward (variant_fwd == GATHER)
    GatherBwdPlan gb;    // the local-gather backward (variant_bwd == GATHER)
};

// Output rows of the sliced tail tiles: y rows b >= first_fwd_row(p), dC rows
// j >= first_dc_row(p).
inline int64_t first_fwd_row(const Plan& p) { return (p.Npad / 256 - p.tail_fwd) * 256; }
inline int64_t first_dc_row(const Plan& p) { return (p.Opad / 256 - p.tail_dc) * 256; }
inline int64_t fwd_tail_rows(const Plan& p) { return p.N - first_fwd_row(p); }
inline int64_t dc_tail_rows(const Plan& p) { return p.O - first_dc_row(p); }

// A k-split: P slices of nks k-tiles each, taken by the last `tail` tile rows.
struct KSplit {
    int P;
    int64_t nks;
    int64_t tail;
};
KSplit k_split(int64_t tiles_m, int64_t tiles_n, int64_t nkt, int64_t rows_out, int64_t row_bytes, int esize);

// Builds the plan; returns KAN_OK or the validation error for `desc` alone.
// materialize = false keeps every basis operand inside the contractions
// (for the fixed-size workspace of kan_forward_static).
int make_plan(const kan_desc_t* desc, Plan* p, bool materialize = true);
// The plan of a 2-D tensor-product layer (always on the matrix cores).
int make_plan_surface(const kan_surface_desc_t* desc, Plan* p);

// The forward pass of a plan built by make_plan, shared by kan_forward and
// kan_forward_static: pointer, alignment, workspace and overlap checks (with
// own_ws the workspace is the library's own array and is not checked), then
// the launches.
int forward_validate(const Plan& p, const void* x, const void* C, const void* W_base, const float* y,
                     const void* ws, size_t ws_bytes, bool own_ws);
int forward_launch(const Plan& p, int flags, const void* x, const void* C, const void* W_base, float* y,
                   void* ws, void* stream);

// ---- launchers (return hipError_t of the launch) ----
// degree 1 .. 5; g built for that degree (t_0 = lo - degree h)
hipError_t launch_basis_eval(const GridK& g, int64_t n, int dtype, const void* x, float* B,
                             float* dB, bool truncated_power, int degree, hipStream_t s);
hipError_t launch_cast_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

hipError_t launch_gather_fwd(const Plan& p, const void* x, const void* C, const void* W,
                             float* y, void* ws, hipStream_t s);
hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void* W,
                            const float* dy, float* dx, void* ws, hipStream_t s);
hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW,
                            void* ws, hipStream_t s);

hipError_t launch_pack_fwd(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s);
hipError_t launch_pack_fwd_sparse(const Plan& p, const void* C, const void* W, void* cp, hipStream_t s);
hipError_t launch_pack_bwd(const Plan& p, const void* C, const void* W, void* cpt, hipStream_t s);
hipError_t launch_prep_dy(const Plan& p, const float* dy, void* dyp, void* dyt, hipStream_t s);
hipError_t launch_mfma_fwd(const Plan& p, const void* x, const void* cp, void* phi, float* ypart, float* y,
                           hipStream_t s);
hipError_t launch_mfma_dx(const Plan& p, const void* x, const void* dyp, const void* cpt,
                          float* part, float* dx, hipStream_t s);
hipError_t launch_mfma_dc(const Plan& p, const void* x, const void* dyt, void* phit, float* cpart, float* dC,
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
