// Reads C ABI calls from stdin, one per line, makes each against the library
// built for the host sanitizers (launchers stubbed, kan_stubs.cpp), and
// prints "<result> <launches>" per call: the status (or the size of a
// *_workspace_size call) and how many launcher stubs the call reached.
// Pointers are plain integers (fake device addresses that the host code
// only compares, or 0 for NULL).
//
//   L fwd|bwd|wsz|prep N I O lo hi G degree dtype base variant flags
//         x C W y dy dx dC dW ws nbytes pass
//   B basis|basis_tp lo hi G degree n dtype x B dB
//   C cast n in out
//   G gfwd|gbwd|gwsz N I groups dtype lo hi G degree x C y dy dx dC ws nbytes
//   S sfwd|sbwd|swsz N P O lo hi G degree dtype flags x C y dy dx dC ws nbytes pass
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kan.h"

extern int g_launches;
extern size_t g_ws_bytes;

static void* P(unsigned long long v) { return reinterpret_cast<void*>(static_cast<uintptr_t>(v)); }

int main() {
    char kind[8], fn[16];
    while (scanf("%7s %15s", kind, fn) == 2) {
        g_launches = 0;
        long long res = 0;
        if (!strcmp(kind, "L")) {
            long long N, I, O;
            float lo, hi;
            int G, deg, dt, base, var, flags, pass;
            unsigned long long x, C, W, y, dy, dx, dC, dW, ws, nb;
            if (scanf("%lld %lld %lld %f %f %d %d %d %d %d %d %llx %llx %llx %llx %llx %llx %llx %llx %llx %llu %d",
                      &N, &I, &O, &lo, &hi, &G, &deg, &dt, &base, &var, &flags, &x, &C, &W, &y, &dy, &dx, &dC,
                      &dW, &ws, &nb, &pass) != 22)
                return 2;
            kan_desc_t d;
            memset(&d, 0, sizeof(d));
            d.N = N, d.I = I, d.O = O, d.grid.lo = lo, d.grid.hi = hi, d.grid.G = G, d.grid.degree = deg;
            d.dtype = dt, d.has_base = base, d.variant = var, d.flags = flags;
            g_ws_bytes = nb;
            if (!strcmp(fn, "fwd")) res = kan_forward(&d, P(x), P(C), P(W), (float*)P(y), P(ws), nb, nullptr);
            else if (!strcmp(fn, "bwd"))
                res = kan_backward(&d, P(x), P(C), P(W), (const float*)P(dy), (float*)P(dx), (float*)P(dC),
                                   (float*)P(dW), P(ws), nb, nullptr);
            else if (!strcmp(fn, "prep")) res = kan_prepare(&d, pass, P(C), P(W), (const float*)P(dy), P(ws), nb, nullptr);
            else res = (long long)kan_workspace_size(&d, pass);
        } else if (!strcmp(kind, "B")) {
            float lo, hi;
            int G, deg, dt;
            long long n;
            unsigned long long x, B, dB;
            if (scanf("%f %f %d %d %lld %d %llx %llx %llx", &lo, &hi, &G, &deg, &n, &dt, &x, &B, &dB) != 9) return 2;
            kan_grid_t g = {lo, hi, G, deg};
            res = !strcmp(fn, "basis") ? kan_basis_eval(&g, n, dt, P(x), (float*)P(B), (float*)P(dB), nullptr)
                                       : kan_basis_eval_tp(&g, n, dt, P(x), (float*)P(B), (float*)P(dB), nullptr);
        } else if (!strcmp(kind, "C")) {
            long long n;
            unsigned long long in, out;
            if (scanf("%lld %llx %llx", &n, &in, &out) != 3) return 2;
            res = kan_cast_f32_to_bf16((const float*)P(in), P(out), n, nullptr);
        } else if (!strcmp(kind, "G")) {
            long long N, I;
            int groups, dt, G, deg;
            float lo, hi;
            unsigned long long x, C, y, dy, dx, dC, ws, nb;
            if (scanf("%lld %lld %d %d %f %f %d %d %llx %llx %llx %llx %llx %llx %llx %llu", &N, &I, &groups, &dt,
                      &lo, &hi, &G, &deg, &x, &C, &y, &dy, &dx, &dC, &ws, &nb) != 16)
                return 2;
            kan_group_desc_t d;
            memset(&d, 0, sizeof(d));
            d.N = N, d.I = I, d.groups = groups, d.dtype = dt, d.grid = {lo, hi, G, deg};
            if (!strcmp(fn, "gfwd")) res = kan_group_forward(&d, P(x), P(C), (float*)P(y), nullptr);
            else if (!strcmp(fn, "gbwd"))
                res = kan_group_backward(&d, P(x), P(C), (const float*)P(dy), (float*)P(dx), (float*)P(dC), P(ws), nb,
                                         nullptr);
            else res = (long long)kan_group_workspace_size(&d);
        } else if (!strcmp(kind, "S")) {
            long long N, Pp, O;
            float lo, hi;
            int G, deg, dt, flags, pass;
            unsigned long long x, C, y, dy, dx, dC, ws, nb;
            if (scanf("%lld %lld %lld %f %f %d %d %d %d %llx %llx %llx %llx %llx %llx %llx %llu %d", &N, &Pp, &O,
                      &lo, &hi, &G, &deg, &dt, &flags, &x, &C, &y, &dy, &dx, &dC, &ws, &nb, &pass) != 18)
                return 2;
            kan_surface_desc_t d;
            memset(&d, 0, sizeof(d));
            d.N = N, d.P = Pp, d.O = O, d.grid = {lo, hi, G, deg}, d.dtype = dt, d.flags = flags;
            g_ws_bytes = nb;
            if (!strcmp(fn, "sfwd")) res = kan_surface_forward(&d, P(x), P(C), (float*)P(y), P(ws), nb, nullptr);
            else if (!strcmp(fn, "sbwd"))
                res = kan_surface_backward(&d, P(x), P(C), (const float*)P(dy), (float*)P(dx), (float*)P(dC), P(ws),
                                           nb, nullptr);
            else res = (long long)kan_surface_workspace_size(&d, pass);
        } else {
            return 2;
        }
        printf("%lld %d\n", res, g_launches);
        fflush(stdout);
    }
    return 0;
}
