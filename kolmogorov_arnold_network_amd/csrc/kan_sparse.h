// Column order and per-span table of the bf16 forward's 2:4 structured-sparse
// basis operand.  Plain integer code, callable from host and device, so that
// the order can be checked on the CPU.
//
// An input's Kb = K + base basis columns (the silu column being c = K) are
// spread over NG groups of 4 logical k: column c goes to group (c + dl) % NG,
// position (c + dl) / NG.  The shift dl = (NG - 1 - K) mod NG with a base
// branch (0 without) puts the silu column at the top position of group
// NG - 1.  With NG >= 4 the 4 consecutive basis functions of a knot span
// (InKAN project page, "Why InKAN?": 4 non-zero functions per span) land in 4
// different groups, so a group holds at most 2 non-zeros: one basis value, and
// the silu value in group NG - 1.
//
// In the operand a group is one dword (its two stored bf16 values, first in
// the low half) plus one index nibble (positions of the two values: first in
// bits 1:0, second in bits 3:2, first < second), the compressed form that
// v_smfmac_f32_32x32x32_bf16 reads.
#pragma once

#include <stdint.h>

namespace kan {

__host__ __device__ inline int sparse_group_shift(int NG, int K, int base) {
    return base ? (NG - 1 - K % NG + NG) % NG : 0;
}

// uint4 words per table entry: NG selectors, the nibbles, the silu mask.
template <int NG>
constexpr int sparse_entry_quads() { return (NG + 5) / 4; }

// Table entry e, dwords w[0 .. 4 * sparse_entry_quads<NG>()):
//   e = sigma + 3 for the first non-zero basis index sigma in [-3, K - 1];
//   e = K + 3: no basis value (x off the extended grid);
//   e = K + 4: the input does not exist (everything zero).
// w[g], g < NG: v_perm_b32 selector that moves group g's basis value out of
//   the packed pairs (b0 b1 : b2 b3) = (bytes 0..3 : bytes 4..7) into the
//   dword half it occupies (selector byte 0x0C yields a zero byte);
// w[NG]: the NG index nibbles;
// w[NG + 1]: mask of the silu half of dword NG - 1 (0 when silu is absent);
// the rest zero.
template <int NG>
__host__ __device__ inline void sparse_table_entry(int e, int K, int base, uint32_t* w) {
    const int dl = sparse_group_shift(NG, K, base);
    const int ps = (K + dl) / NG;                               // the silu column's position
    uint32_t nib = NG == 8 ? 0x44444444u : (0x44444444u & ((1u << (4 * NG)) - 1));
    for (int g = 0; g < NG; ++g) w[g] = 0x0C0C0C0Cu;
    bool silu_group_taken = false;
    if (e <= K + 2) {
        for (int r = 0; r < 4; ++r) {
            const int m = e - 3 + r;
            if (m < 0 || m >= K) continue;
            const int g = (m + dl) % NG, p = (m + dl) / NG;
            const uint32_t lo = 0x0C0C0000u | ((2u * r + 1) << 8) | (2u * r);
            const uint32_t hi = 0x00000C0Cu | ((2u * r + 1) << 24) | ((2u * r) << 16);
            uint32_t v;
            if (base && g == NG - 1) {                          // below the silu value
                w[g] = lo;
                v = (uint32_t)((ps << 2) | p);
                silu_group_taken = true;
            } else if (p == 0) {
                w[g] = lo;
                v = 4u;
            } else {
                w[g] = hi;
                v = (uint32_t)(p << 2);
            }
            nib = (nib & ~(0xFu << (4 * g))) | (v << (4 * g));
        }
    }
    const bool silu = base && e <= K + 3;
    if (silu && !silu_group_taken)                              // silu alone, in the high half
        nib = (nib & ~(0xFu << (4 * (NG - 1)))) | ((uint32_t)(ps << 2) << (4 * (NG - 1)));
    w[NG] = nib;
    w[NG + 1] = silu ? 0xFFFF0000u : 0u;
    for (int k = NG + 2; k < 4 * sparse_entry_quads<NG>(); ++k) w[k] = 0;
}

}  // namespace kan
