// Host check of the sparse forward's column order and per-span table
// (kan_sparse.h): for every (K, base) the library accepts for the sparse form
// and every table entry, a block is assembled the way the kernel assembles it
// (one v_perm_b32 per dword, silu or-ed into the last dword under the mask),
// decompressed through the index nibbles, and compared with the dense basis
// row of that span placed in the column order the coefficient packing uses.
// v_perm_b32 is emulated from the instruction's documented byte-select
// semantics: selector bytes 0-3 pick bytes of the second source, 4-7 bytes of
// the first, 12 gives 0x00.
#define __host__
#define __device__
#include "kan_sparse.h"

#include <cstdio>

using namespace kan;

static uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
    const uint64_t v = ((uint64_t)s0 << 32) | s1;
    uint32_t r = 0;
    for (int k = 0; k < 4; ++k) {
        const uint32_t b = (sel >> (8 * k)) & 0xFF;
        uint32_t o;
        if (b < 8) o = (uint32_t)(v >> (8 * b)) & 0xFF;
        else if (b == 12) o = 0;
        else return 0xDEADBEEFu;                                 // no other selector is used
        r |= o << (8 * k);
    }
    return r;
}

template <int NG>
static int check(int K, int base) {
    const int dl = sparse_group_shift(NG, K, base), Kb = K + base;
    int bad = 0;
    // the packing reads column c = p NG + g - dl at (group g, position p):
    // the same bijection, inside the input's 4 NG logical columns
    for (int c = 0; c < Kb; ++c) {
        const int g = (c + dl) % NG, p = (c + dl) / NG;
        if (p >= 4 || p * NG + g - dl != c) ++bad;
    }
    for (int e = 0; e <= K + 4; ++e) {
        uint32_t w[4 * sparse_entry_quads<NG>()];
        sparse_table_entry<NG>(e, K, base, w);
        // distinct tags stand for b0..b3 and silu
        const uint32_t tag[4] = {0x1001, 0x1002, 0x1003, 0x1004}, sil = 0x2005;
        const uint32_t p01 = tag[0] | tag[1] << 16, p23 = tag[2] | tag[3] << 16;
        uint32_t d[NG];
        for (int g = 0; g < NG; ++g) d[g] = perm(p23, p01, w[g]);
        d[NG - 1] |= (sil << 16) & w[NG + 1];
        uint32_t got[NG][4] = {}, want[NG][4] = {};
        for (int g = 0; g < NG; ++g) {
            const uint32_t nib = (w[NG] >> (4 * g)) & 15, f = nib & 3, s = nib >> 2;
            if (f >= s) { ++bad; continue; }
            got[g][f] = d[g] & 0xFFFF;
            got[g][s] = d[g] >> 16;
        }
        const int sig = e - 3;
        for (int c = 0; c < Kb; ++c) {
            uint32_t v = 0;
            if (c < K && e <= K + 2 && c >= sig && c <= sig + 3) v = tag[c - sig];
            if (c == K && base && e <= K + 3) v = sil;
            want[(c + dl) % NG][(c + dl) / NG] = v;
        }
        for (int g = 0; g < NG; ++g)
            for (int p = 0; p < 4; ++p)
                if (got[g][p] != want[g][p]) {
                    if (bad < 5)
                        printf("mismatch NG=%d K=%d base=%d e=%d group %d position %d: %x, want %x\n", NG,
                               K, base, e, g, p, got[g][p], want[g][p]);
                    ++bad;
                }
    }
    return bad;
}

int main() {
    int cases = 0, bad = 0;
    for (int base = 0; base <= 1; ++base)
        for (int K = 4; K <= 40; ++K) {
            // the planner's rule for the sparse form (bf16, no dense flag)
            const int Kb = K + base;
            int ng = (Kb + 3) / 4 > 4 ? (Kb + 3) / 4 : 4;
            ng += ng & 1;
            if (!(ng <= 8 && Kb >= 11 && 8 * ng <= 3 * Kb)) continue;
            ++cases;
            bad += ng == 4 ? check<4>(K, base) : ng == 6 ? check<6>(K, base) : check<8>(K, base);
        }
    printf("cases %d mismatches %d\n", cases, bad);
    return bad != 0;
}
