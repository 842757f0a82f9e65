// Launcher stubs for the host-only sanitizer build of the C ABI: the
// validation and planning code of kan_api.cpp and kan_plan.cpp is compiled
// with AddressSanitizer and UndefinedBehaviorSanitizer and linked against
// these instead of the GPU kernels.  Each stub counts its call and checks the
// arguments every launcher relies on (non-null required pointers, workspace
// carve-outs inside the workspace the caller declared), so that a call which
// fails validation can be seen to reach no launcher.
#include <stdio.h>
#include <stdlib.h>

#include "kan_internal.h"

int g_launches = 0;
size_t g_ws_bytes = 0;          // bytes of workspace the driver declared for the current call

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace kan {

static void need(bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "stub check failed: %s\n", what);
        abort();
    }
}
static void in_ws(size_t off, size_t bytes, const void* ws) {
    if (bytes == 0) return;
    need(ws != nullptr, "workspace pointer");
    need(off + bytes <= g_ws_bytes, "workspace carve-out inside the declared workspace");
}

hipError_t launch_basis_eval(const GridK&, int64_t n, int, const void* x, float* B, float* dB, bool, int degree,
                             hipStream_t) {
    need(n > 0 && x && (B || dB) && degree >= 1 && degree <= 5, "basis arguments");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_cast_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t) {
    need(in && out && n > 0, "cast arguments");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t) {
    need(p && n >= 0, "fill arguments");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gather_fwd(const Plan& p, const void* x, const void* C, const void*, float* y, void* ws,
                             hipStream_t) {
    need(x && C && y && p.N > 0, "gather forward pointers");
    need(p.gf.ic >= 1 && p.gf.ic <= 8 && p.gf.split >= 1 && p.gf.is >= 1, "gather forward plan");
    in_ws(0, p.gf.ws, ws);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gather_dx(const Plan& p, const void* x, const void* C, const void*, const float* dy, float* dx,
                            void* ws, hipStream_t) {
    need(x && C && dy && dx && p.N > 0, "gather dx pointers");
    if (p.gb.sx > 1) in_ws(p.gb.off_dxp, (size_t)p.gb.sx * p.N * p.I * 4, ws);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gather_dc(const Plan& p, const void* x, const float* dy, float* dC, float* dW, void* ws,
                            hipStream_t) {
    need(x && dy && (dC || dW) && p.N > 0, "gather dC pointers");
    if (p.gb.sc > 1) {
        if (dC) in_ws(p.gb.off_dcp, (size_t)p.gb.sc * p.O * p.I * p.K * 4, ws);
        if (dW) in_ws(p.gb.off_dwp, (size_t)p.gb.sc * p.O * p.I * 4, ws);
    }
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_pack_fwd(const Plan& p, const void* C, const void*, void* cp, hipStream_t) {
    need(C && cp, "pack pointers");
    need(p.sz_cp > 0, "pack size");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_pack_fwd_sparse(const Plan& p, const void* C, const void*, void* cp, hipStream_t) {
    need(C && cp && p.sparse, "sparse pack");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_pack_bwd(const Plan& p, const void* C, const void*, void* cpt, hipStream_t) {
    need(C && cpt && p.sz_cpt > 0, "backward pack");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prep_dy(const Plan&, const float* dy, void* dyp, void* dyt, hipStream_t) {
    need(dy && dyp && dyt, "dy pointers");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_mfma_fwd(const Plan& p, const void* x, const void* cp, void* phi, float* ypart, float* y,
                           hipStream_t) {
    need(x && cp && y && (!p.mat_fwd || phi), "mfma forward pointers");
    if (p.mat_fwd) need(p.off_phi + (size_t)p.Npad * p.Kf * 2 <= p.ws_fwd && !p.sparse, "forward basis in the workspace");
    need(p.split_fwd >= 1 && (p.split_fwd == 1 || ypart), "mfma forward slices");
    need(p.split_fwd == 1 || (p.tail_fwd >= 1 && p.tail_fwd <= p.Npad / 256 && fwd_tail_rows(p) >= 1 &&
                              p.nks_fwd * (p.split_fwd - 1) < (p.sparse ? p.Kfs / 64 : p.Kf / p.BK)),
         "mfma forward tail");
    if (p.split_fwd > 1)
        need(p.off_yp + (size_t)p.split_fwd * fwd_tail_rows(p) * p.O * 4 <= p.ws_fwd, "forward partials in the workspace");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_mfma_dx(const Plan&, const void* x, const void* dyp, const void* cpt, float* part, float* dx,
                          hipStream_t) {
    need(x && dyp && cpt && part && dx, "mfma dx pointers");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_mfma_dc(const Plan& p, const void* x, const void* dyt, void* phit, float* cpart, float*, float*,
                          hipStream_t) {
    need(x && dyt && (p.split_dc == 1 || cpart) && (!p.mat_dc || phit), "mfma dC pointers");
    if (p.mat_dc)
        need(p.off_phit + (size_t)p.tiles_dx * 256 * p.Npad * 2 <= p.ws_bwd && (p.Kb <= 12 || p.pair), "dC basis in the workspace");
    need(p.split_dc == 1 || (p.tail_dc >= 1 && p.tail_dc <= p.Opad / 256 && dc_tail_rows(p) >= 1 &&
                             p.nks_dc * (p.split_dc - 1) < p.Npad / p.BK),
         "mfma dC tail");
    if (p.split_dc > 1)
        need(p.off_dcp + (size_t)p.split_dc * dc_tail_rows(p) * p.I * p.Kb * 4 <= p.ws_bwd, "dC partials in the workspace");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_grouped_fwd(const GridK&, int64_t N, int64_t I, int groups, int, const void* x, const void* C,
                              float* y, hipStream_t) {
    need(N > 0 && I > 0 && groups >= 1 && x && C && y, "grouped forward");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_grouped_bwd(const GridK&, int64_t N, int64_t I, int groups, int, const void*, const void* C,
                              const float*, float*, float* dC, float* part, float* red, hipStream_t) {
    need(I > 0 && groups >= 1 && C, "grouped backward");
    need(!dC || N == 0 || (part && red), "grouped backward workspace");
    ++g_launches;
    return hipSuccess;
}

}  // namespace kan
