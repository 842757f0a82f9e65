/*
 * kan.h - C ABI of the MI355X (gfx950) B-spline KAN layer library.
 *
 * The layer (InKAN project page, "What is a KAN?"): every edge (j, i) carries a
 * learned cubic B-spline phi_ji, and output j sums them over the inputs,
 *
 *     y[b, j] = sum_i sum_m C[j, i, m] * B_m(x[b, i])
 *             + has_base * sum_i W_base[j, i] * silu(x[b, i]),
 *
 * with B_m, m = 0 .. G+2, the uniform cubic B-splines of a grid of G equal
 * intervals on [lo, hi] extended by 3 knots on each side (knots
 * t_r = lo + (r - 3) h, h = (hi - lo) / G, r = 0 .. G+6).  The residual
 * W_base * silu(x) branch is optional and is not on the pages.  Training
 * backward ("same optimizer, same training loop", InKAN page, "Why InKAN?"):
 *
 *     dx[b, i]      = sum_j dy[b, j] * (sum_m C[j, i, m] * B'_m(x[b, i])
 *                                       + W_base[j, i] * silu'(x[b, i]))
 *     dC[j, i, m]   = sum_b dy[b, j] * B_m(x[b, i])
 *     dW_base[j, i] = sum_b dy[b, j] * silu(x[b, i])
 *
 * An input outside the extended grid [t_0, t_{G+6}) has every B_m = 0 and
 * contributes through the base branch only; the layer never clamps x.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Layouts are row-major and contiguous: x [N, I]; C [O, I, G+3] with m
 *   fastest; W_base [O, I]; y, dy [N, O]; dx [N, I]; dC [O, I, G+3];
 *   dW_base [O, I].
 * - x, C and W_base share one storage dtype (KAN_F32 or KAN_BF16); y, dy, dx,
 *   dC and dW_base are always float32.  Arithmetic accumulates in float32
 *   (the float32 forwards add their partial sums in float64; see
 *   kan_variant_t).
 * - Tensor pointers are DEVICE pointers, 16-byte aligned.  `desc` and `grid`
 *   are HOST pointers, read during the call only.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *   is enqueued asynchronously on it; nothing synchronises the host.
 * - The caller owns every buffer.  The library allocates and frees no device
 *   memory and keeps no pointer after returning.  Scratch space is the
 *   caller's workspace of at least kan_workspace_size() bytes, 256-byte aligned.
 * - Outputs are overwritten, never accumulated into.  Outputs must not overlap
 *   inputs or each other (KAN_ERR_ALIAS).
 * - Every argument is validated before any device work: a call that returns
 *   an error has enqueued nothing.  A launch failure returns KAN_ERR_HIP.
 * - Results are deterministic: the same inputs give bitwise-identical outputs
 *   on every call (no floating-point atomics anywhere).
 * - The library holds no mutable global state; concurrent calls on different
 *   streams with disjoint outputs are safe.
 * - Every call only enqueues kernels on `stream` (zero fills are kernels, no
 *   memset or copy nodes), so a call may be captured into a HIP graph, with
 *   its workspace allocated beforehand, and the graph replayed.
 */
#ifndef KAN_H
#define KAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KAN_ABI_VERSION 1

typedef enum {
    KAN_OK = 0,
    KAN_ERR_NULL = -1,        /* a required pointer is NULL, or a forbidden one is not */
    KAN_ERR_SHAPE = -2,       /* N < 0, I < 1, O < 1, or a size beyond the index range: N, O,
                               * 2P and a row's I*(G+D+has_base) columns must each stay below
                               * 2^31 - 4096 (whole tensors may exceed 2^31 elements; addresses
                               * are 64-bit); the basis entry points bound n*K the same way */
    KAN_ERR_GRID = -3,        /* G < 1 or G > 125 (2-D layer: 13), lo >= hi, or lo / hi not finite */
    KAN_ERR_DTYPE = -4,       /* dtype not KAN_F32 / KAN_BF16 */
    KAN_ERR_ALIGN = -5,       /* a tensor pointer not 16-byte aligned (workspace: 256) */
    KAN_ERR_WORKSPACE = -6,   /* workspace smaller than kan_workspace_size() */
    KAN_ERR_HIP = -7,         /* a HIP launch failed */
    KAN_ERR_UNSUPPORTED = -8, /* degree outside what the entry point takes, bad variant / has_base / pass / flags */
    KAN_ERR_ALIAS = -9        /* an output overlaps an input or another output */
} kan_status_t;

typedef enum { KAN_F32 = 0, KAN_BF16 = 1 } kan_dtype_t;

/* Kernel family.  MFMA runs the contraction over the dense basis
 * (I*(G+D+has_base) wide) on the matrix cores, with the basis generated in LDS
 * and never written to memory; it needs G+D+has_base <= 256, and at least 4
 * for a degree D other than 3.  A float32 MFMA forward adds its contraction
 * in fixed slices of at most 256 (i, m) terms whose float32 partial sums are
 * added in float64, so that its rounding stays small enough for a following
 * layer's B' (which amplifies it about tenfold) to keep a chain of layers
 * within 1e-5.  GATHER touches only the D+1 non-zero basis functions per input
 * (InKAN page, "Why InKAN?": local 4-basis lookup) on the vector ALUs; its
 * forward adds the partial sums of chunks of at most 8 inputs in float64.
 * AUTO picks per pass: bf16 runs both passes on MFMA; float32 runs the forward
 * on GATHER and the backward on whichever family is estimated faster: GATHER
 * (about N*I*O / 1.6e12 s, independent of G) or MFMA (about
 * 4*N*I*O*(G+D+has_base) / 110e12 s + 150 us), that is GATHER for small
 * layers and from about 17 columns per input up; GATHER wherever MFMA does
 * not fit. */
typedef enum { KAN_VARIANT_AUTO = 0, KAN_VARIANT_MFMA = 1, KAN_VARIANT_GATHER = 2 } kan_variant_t;

typedef enum { KAN_PASS_FORWARD = 0, KAN_PASS_BACKWARD = 1 } kan_pass_t;

/* Grid: G intervals on [lo, hi], 1 <= G <= 125 (the G+D coefficients of an
 * input for a tile of outputs are staged in LDS), and the spline degree.  The
 * pages' layer is cubic (InKAN page) and 3 is the default everywhere; the
 * layer also takes degree D = 1 .. 5 (FlashKAN page: the degree-k form of the
 * basis), with the grid extended by D knots on each side (t_r = lo + (r - D) h)
 * and K = G + D coefficients per edge, so C is [O, I, G+D] and the formulas
 * at the top hold with B_m of degree D.  Every variant takes every degree,
 * except that MFMA needs G + D + has_base >= 4 when D != 3 and the
 * structured-sparse forward is cubic only.  The grouped activation and the
 * 2-D layer are cubic only. */
typedef struct {
    float lo;
    float hi;
    int32_t G;
    int32_t degree;
} kan_grid_t;

/* One layer.  N rows may be 0 (forward and dx are then no-ops; dC and dW_base
 * are filled with zeros). */
typedef struct {
    int64_t N;
    int64_t I;
    int64_t O;
    kan_grid_t grid;
    int32_t dtype;     /* kan_dtype_t: storage of x, C, W_base */
    int32_t has_base;  /* 0 or 1 */
    int32_t variant;   /* kan_variant_t */
    int32_t flags;     /* 0, or KAN_FLAG_PREPARED, KAN_FLAG_DENSE_FORWARD, KAN_FLAG_TP_FORWARD */
} kan_desc_t;

/* The workspace already holds this pass's packed operands, written by
 * kan_prepare (or by the last kan_forward / kan_backward without this flag)
 * for the same desc, C, W_base (and dy, for the backward pass); the call then
 * skips packing and launches only the contraction kernels.  The caller must
 * not have changed those inputs since. */
#define KAN_FLAG_PREPARED 1

/* The MFMA forward of a bf16 layer with 11 <= G+3+has_base <= 32 runs by
 * default on the structured-sparse matrix instructions: every input's
 * G+3+has_base basis columns are permuted so that any 4 consecutive basis
 * functions (the non-zero ones of a knot span; InKAN page, "Why InKAN?") and
 * the silu column fall at most 2 to a group of 4, and the 2:4-sparse basis
 * tile is multiplied at twice the dense rate.  The result is the same sum in
 * a different order.  This flag asks for the dense basis instead.  It may be
 * combined with KAN_FLAG_PREPARED; both passes of a prepared pair must agree
 * on it. */
#define KAN_FLAG_DENSE_FORWARD 2

/* The dense bf16 forward on the matrix cores (implies KAN_FLAG_DENSE_FORWARD)
 * with its basis tile generated by the truncated-power form instead of the
 * knot span (FlashKAN project page: a degree-k B-spline is a combination of
 * k+2 shifted truncated powers of the normalised coordinate, clamped to
 * [0, k+1]): every column (i, m) of the tile is B(x/h + shift - m) on its own,
 * with no span lookup, zero fill or scatter.  The values are rounded to bf16
 * like the span form's (their float32 cancellation error, ~1e-6, is far
 * below bf16's rounding).  Only for bf16 storage, degree 3, and a forward
 * that runs on MFMA (KAN_ERR_UNSUPPORTED otherwise); both passes of a
 * prepared pair must agree on it.  It costs G+3+has_base basis evaluations
 * per (row, input) where the span form costs one, and on MI355X, whose bf16
 * matrix rate is 16x its vector float32 rate, that vector work outlasts the
 * contraction: the forward is 2.5x to 8x slower than the span form.  It is
 * an independent construction of the same operand, not a fast path. */
#define KAN_FLAG_TP_FORWARD 4

/* KAN_ABI_VERSION of the loaded library. */
int kan_abi_version(void);

/* Static description of a status code (never NULL). */
const char* kan_status_string(int status);

/* Bytes of workspace a pass needs (SIZE_MAX if `desc` is invalid).  `pass`
 * is kan_pass_t.  On MFMA it holds the packed operands of kan_prepare and the
 * float32 partial outputs of k-range slices (the forward's y, slices of at
 * most 256 terms in float32 and otherwise where too few output tiles fill
 * the GPU; dC and dW_base over batch slices), which are added in slice
 * order.  A bf16 layer with few columns per input (G + 3 + has_base <= 12)
 * also gets its dense basis built once from x, in bf16, when enough output
 * tiles read it: the forward's [N][I*(G+3+has_base)] from O > 1792, dC's
 * transpose from O > 512 (the 2-D layer's dC pair basis too), each at most
 * 1 GiB.  kan_forward writes it; it is not part of kan_prepare.  GATHER needs it only when too few blocks fill the GPU: the
 * forward then splits its inputs into slices whose float64 partial outputs
 * [slices][N][O] are added in slice order, the backward splits dx over
 * output slices and dC / dW_base over row slices, with float32 partials
 * added in slice order (in float64). */
size_t kan_workspace_size(const kan_desc_t* desc, int pass);

/* Packs what a pass reads into the workspace: for a pass on MFMA the
 * coefficient operand C' = [C | W_base] per input, zero-padded to the tile
 * grid (forward: [O][I*(G+3+has_base)], or the structured-sparse column order
 * described at KAN_FLAG_DENSE_FORWARD; backward: the transpose of the dense
 * form), and for the backward pass also dy rounded to the storage dtype in
 * both orientations.  dy may be NULL for the forward pass.  A no-op for a
 * pass on GATHER. */
int kan_prepare(const kan_desc_t* desc, int pass, const void* C, const void* W_base,
                const float* dy, void* workspace, size_t workspace_bytes, void* stream);

/* Forward: y [N, O] float32.  x, C, W_base in desc->dtype; W_base must be NULL
 * exactly when has_base == 0. */
int kan_forward(const kan_desc_t* desc, const void* x, const void* C, const void* W_base,
                float* y, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Forward without a caller workspace --------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * forward as kan_forward (the same bits), with the workspace taken from a
 * fixed array of KAN_STATIC_SCRATCH_BYTES of device memory inside the
 * library.  It never builds the basis in the workspace (kan_workspace_size);
 * its contraction generates the same basis tiles on chip.  Every GPU the
 * library runs on holds its own copy of that array from the first call
 * until the process ends; the call itself allocates and frees nothing.  A
 * layer whose forward workspace, without the built basis, is larger returns
 * KAN_ERR_WORKSPACE before any work; KAN_FLAG_PREPARED is
 * refused (KAN_ERR_UNSUPPORTED).  The array keeps the last call's contents
 * and nothing in it has to start at zero.  All calls on one GPU share the
 * array, so calls that overlap in time on one GPU (on different streams or
 * from different threads) race and must be ordered by the caller; calls
 * queued on one stream are ordered by the stream.  `stream` must belong to
 * the current device.  Other arguments, validation and errors as for
 * kan_forward. */
#define KAN_STATIC_SCRATCH_BYTES (32u << 20)
int kan_forward_static(const kan_desc_t* desc, const void* x, const void* C, const void* W_base,
                       float* y, void* stream);

/* Backward.  dy [N, O] float32 in.  dx [N, I], dC [O, I, G+3] and dW_base
 * [O, I] are float32 outputs; each may be NULL to skip it (dW_base must be
 * NULL when has_base == 0).  dC and dW_base are sums over all N rows, reduced
 * in a fixed order without atomics (FlashKAT abstract: atomic gradient
 * accumulation is what slows the backward pass); when there are too few
 * output tiles, over fixed batch slices whose partial sums are then added in
 * slice order. */
int kan_backward(const kan_desc_t* desc, const void* x, const void* C, const void* W_base,
                 const float* dy, float* dx, float* dC, float* dW_base,
                 void* workspace, size_t workspace_bytes, void* stream);

/* The span / local-basis step on its own, for checking the device basis.
 * x [n] in `dtype`; B and dB [n, G+D] float32 outputs (either may be NULL),
 * D = grid->degree: B[k, m] = B_m(x[k]) and dB[k, m] = dB_m/dx(x[k]), computed
 * from the D+1 non-zero pieces of the knot span that holds x[k] (InKAN page,
 * "Why InKAN?": stable piecewise evaluation, local basis lookup) and written
 * densely.  Here the degree may be 1 .. 5 (the layer entry points take 3):
 * the grid is extended by D knots on each side (t_r = lo + (r - D) h), and
 * for D != 3 the pieces come from the uniform-knot recurrence
 * N^q_r = ((u + q - r) N^{q-1}_{r-1} + (r + 1 - u) N^{q-1}_r) / q, whose
 * terms are non-negative. */
int kan_basis_eval(const kan_grid_t* grid, int64_t n, int dtype, const void* x,
                   float* B, float* dB, void* stream);

/* The same dense B and dB from the truncated-power form instead (FlashKAN
 * project page: a degree-k B-spline is a combination of k+2 shifted
 * (x)_+^k terms, with the normalised coordinate clamped to [0, k+1]):
 * u = (x[k] - t_m) / h clamped to [0, D+1],
 *     B_m = sum_i (-1)^i C(D+1, i) (u-i)_+^D / D!,
 *     dB_m/dx = sum_i (-1)^i C(D+1, i) (u-i)_+^(D-1) / ((D-1)! h),
 * at D = 3: B_m = (u^3 - 4 (u-1)_+^3 + 6 (u-2)_+^3 - 4 (u-3)_+^3) / 6.  At D = 1
 * the derivative's step terms take the unclamped u with (w)_+^0 = [w >= 0].
 * Every (k, m) is evaluated on its own, with no span lookup.  The alternating
 * sum cancels near u = 4, so in float32 it is less accurate than
 * kan_basis_eval (absolute error up to ~1e-5 at D = 3, more at higher degree,
 * and values may round slightly below 0, where the local form cannot; InKAN
 * page, "Why InKAN?").  Arguments,
 * validation and errors as for kan_basis_eval. */
int kan_basis_eval_tp(const kan_grid_t* grid, int64_t n, int dtype, const void* x,
                      float* B, float* dB, void* stream);

/* ---- Grouped spline activation ------------------------------------------
 * The element-wise form of the edge function: every channel of a row passes
 * through one learned cubic B-spline, shared by a group of consecutive
 * channels (InKAN project page: per-coordinate spline curves; FlashKAT
 * abstract: grouped KAN activations, whose training is held back by the
 * atomic accumulation of the coefficient gradient),
 *
 *     y[b, i]  = sum_m C[g(i), m] * B_m(x[b, i]),    g(i) = floor(i * groups / I),
 *     dx[b, i] = dy[b, i] * sum_m C[g(i), m] * B'_m(x[b, i]),
 *     dC[g, m] = sum_b sum_{i : g(i) = g} dy[b, i] * B_m(x[b, i]),
 *
 * with B_m the basis of the layer (grid as for kan_desc_t).  Layouts: x, y,
 * dy, dx [N, I]; C, dC [groups, G+3], m fastest.  x and C in `dtype`; y, dy,
 * dx and dC float32.  The conventions of the layer entry points hold
 * (device pointers 16-byte aligned, outputs overwritten, no overlap,
 * validation before any work, deterministic results). */
typedef struct {
    int64_t N;          /* rows, >= 0 */
    int64_t I;          /* channels, >= 1 */
    int32_t groups;     /* 1 <= groups <= I; groups == I: one spline per channel */
    int32_t dtype;      /* kan_dtype_t: storage of x and C */
    kan_grid_t grid;
} kan_group_desc_t;

/* Bytes of workspace kan_group_backward needs for dC (SIZE_MAX if `desc` is
 * invalid): the per-channel sums of fixed chunks of rows, then their sum over
 * the chunks, which the groups' channels are added from (no atomics). */
size_t kan_group_workspace_size(const kan_group_desc_t* desc);

/* Forward: y [N, I] float32. */
int kan_group_forward(const kan_group_desc_t* desc, const void* x, const void* C, float* y,
                      void* stream);

/* Backward: dy [N, I] in; dx [N, I] and dC [groups, G+3] out, either may be
 * NULL to skip it.  The workspace (256-byte aligned) is needed only with dC.
 * N = 0 fills dC with zeros. */
int kan_group_backward(const kan_group_desc_t* desc, const void* x, const void* C, const float* dy,
                       float* dx, float* dC, void* workspace, size_t workspace_bytes, void* stream);

/* ---- 2-D tensor-product spline layer ---------------------------------------
 * Beside univariate spline layers, the InKAN project page ("1D and 2D
 * Splines") offers tensor-product B-spline surfaces for approximating a
 * function of two inputs jointly.  Here the inputs of a row are taken in
 * consecutive pairs (x[b, 2p], x[b, 2p+1]), p = 0 .. P-1, every (output j,
 * pair p) edge carries one bicubic surface over the layer's 1-D basis, and
 * output j sums its edges:
 *
 *     y[b, j] = sum_p sum_{m,n} C[j, p, m, n] * B_m(x[b, 2p]) * B_n(x[b, 2p+1]),
 *
 * at most 16 non-zero products per (row, pair).  Backward with dy [N, O]:
 *
 *     dx[b, 2p]      = sum_j dy[b, j] sum_{m,n} C[j, p, m, n] B'_m(x[b, 2p]) B_n(x[b, 2p+1])
 *     dx[b, 2p+1]    = sum_j dy[b, j] sum_{m,n} C[j, p, m, n] B_m(x[b, 2p]) B'_n(x[b, 2p+1])
 *     dC[j, p, m, n] = sum_b dy[b, j] B_m(x[b, 2p]) B_n(x[b, 2p+1])
 *
 * Layouts: x, dx [N, 2P]; C, dC [O, P, G+3, G+3] with n fastest; y, dy
 * [N, O].  x and C in `dtype`, the rest float32.  Both passes run on the
 * matrix cores over the (G+3)^2 products per pair, generated in LDS; a pair's
 * columns must fit one 256-wide tile, so 1 <= G <= 13.  The conventions of
 * the layer entry points hold (device pointers 16-byte aligned, workspace
 * 256-byte aligned and caller-owned, outputs overwritten, no overlap,
 * validation before any work, deterministic results; N = 0 fills dC with
 * zeros). */
typedef struct {
    int64_t N;          /* rows, >= 0 */
    int64_t P;          /* input pairs, >= 1 (x has 2P columns) */
    int64_t O;          /* outputs, >= 1 */
    kan_grid_t grid;    /* 1 <= G <= 13, degree 3 */
    int32_t dtype;      /* kan_dtype_t: storage of x and C */
    int32_t flags;      /* 0, or KAN_FLAG_PREPARED: the workspace holds this
                           pass's packed operands from the last call without
                           the flag (same desc, C, and dy for the backward);
                           and/or KAN_FLAG_DENSE_FORWARD (below) */
} kan_surface_desc_t;

/* With bf16 storage and G = 5 the forward of the 2-D layer runs on the
 * structured-sparse matrix instructions: within each m-row of a pair's 8 x 8
 * columns the n index is permuted into two groups of 4 by parity, so the 4
 * consecutive n of a span put 2 values in each group, and the 2:4-sparse tile
 * is multiplied at twice the dense rate.  KAN_FLAG_DENSE_FORWARD asks for the
 * dense form; both passes of a prepared pair must agree on it. */

/* Bytes of workspace a pass of the 2-D layer needs (SIZE_MAX if `desc` is
 * invalid): the packed coefficient operand, and for the backward dy in both
 * orientations and the dx partial sums of pairs cut by a tile edge, plus the
 * float32 partial outputs of k-range slices and, for a bf16 backward with
 * O > 512, dC's pair basis built once, as for kan_workspace_size. */
size_t kan_surface_workspace_size(const kan_surface_desc_t* desc, int pass);

/* Forward: y [N, O] float32. */
int kan_surface_forward(const kan_surface_desc_t* desc, const void* x, const void* C, float* y,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Backward: dx [N, 2P] and dC [O, P, G+3, G+3], float32; either may be NULL
 * to skip it.  dC is reduced over all rows in a fixed order without atomics. */
int kan_surface_backward(const kan_surface_desc_t* desc, const void* x, const void* C,
                         const float* dy, float* dx, float* dC, void* workspace,
                         size_t workspace_bytes, void* stream);

/* float32 -> bfloat16, round to nearest even (NaN stays NaN).  n elements;
 * `out` receives the 16-bit patterns.  Used between bf16 layers, where a
 * float32 layer output becomes the next layer's bf16 input. */
int kan_cast_f32_to_bf16(const float* in, void* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KAN_H */
