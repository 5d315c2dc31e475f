// NF4 level table and the register lookup that dequantizes eight 4-bit NF4
// codes into fp16 levels (Quantization operators guide §3.4), shared by the
// NF4 decode GEMV and the NF4 form of the large-M GEMM (gfx950).
#pragma once

#include "q4_internal.hpp"

namespace q4k {

// The guide's levels: Phi^-1((i + 0.5) / 16) / Phi^-1(31 / 32), rounded to
// fp16, ascending (bit patterns).
inline constexpr uint16_t kNf4Levels[16] = {0xBC00, 0xB9A9, 0xB856, 0xB6AB, 0xB4F9, 0xB2E9, 0xB013, 0xA963,
                                            0x2963, 0x3013, 0x32E9, 0x34F9, 0x36AB, 0x3856, 0x39A9, 0x3C00};

// magnitude tables: entry j (0..7) is |level[8 + j]|; low bytes and high bytes
// of the fp16 patterns, 8 bytes each, as two dwords (v_perm_b32 sources)
constexpr uint32_t nf4_lo_bytes(int d)
{
    uint32_t v = 0;
    for (int b = 0; b < 4; b++) v |= (uint32_t)(kNf4Levels[8 + 4 * d + b] & 0xFF) << (8 * b);
    return v;
}
constexpr uint32_t nf4_hi_bytes(int d)
{
    uint32_t v = 0;
    for (int b = 0; b < 4; b++) v |= (uint32_t)(kNf4Levels[8 + 4 * d + b] >> 8) << (8 * b);
    return v;
}
constexpr uint32_t kNf4Lo0 = nf4_lo_bytes(0), kNf4Lo1 = nf4_lo_bytes(1), kNf4Hi0 = nf4_hi_bytes(0),
                   kNf4Hi1 = nf4_hi_bytes(1);

// 8 codes (one dword, code i in nibble i) -> their 8 fp16 levels as 4 dwords
// of pairs, in the k order 0, 2, 4, 6, 1, 3, 5, 7 (codes 0, 2 in dword 0,
// 4, 6 in dword 1, 1, 3 in dword 2, 5, 7 in dword 3): the order the lookup
// produces them in, for callers that store X in the same order.
// Magnitude index j: 7 - c below 8 (negative levels), c - 8 from 8 up; with
// b8 the code's bit 3 (8 or 0 per nibble), b8 - b8 / 8 is 7 or 0, and
// ~(c ^ that) & 7 is j. The sign bit of a negative level is set from ~bit 3.
__device__ __forceinline__ u32x4 nf4_levels8_kperm(uint32_t d)
{
    const uint32_t b8 = d & 0x88888888u;
    const uint32_t t = b8 - (b8 >> 3);
    // v_bitop3 (bit (a << 2 | b << 1 | c) of the table is f(a, b, c)):
    // 0x82 is ~(a ^ b) & c, 0xF2 is a | (~b & c). Written out as builtins so
    // the compiler keeps the mask before the shift and the NOT inside.
    const uint32_t jA = __builtin_amdgcn_bitop3_b32(d, t, 0x07070707u, 0x82);        // codes 0, 2, 4, 6
    const uint32_t jB = __builtin_amdgcn_bitop3_b32(d, t, 0x70707070u, 0x82) >> 4;   // codes 1, 3, 5, 7
    const uint32_t loA = __builtin_amdgcn_perm(kNf4Lo1, kNf4Lo0, jA), loB = __builtin_amdgcn_perm(kNf4Lo1, kNf4Lo0, jB);
    const uint32_t hiA = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(kNf4Hi1, kNf4Hi0, jA), d << 4, 0x80808080u, 0xF2);
    const uint32_t hiB = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(kNf4Hi1, kNf4Hi0, jB), d, 0x80808080u, 0xF2);
    return u32x4{__builtin_amdgcn_perm(hiA, loA, 0x05010400u), __builtin_amdgcn_perm(hiA, loA, 0x07030602u),
                 __builtin_amdgcn_perm(hiB, loB, 0x05010400u), __builtin_amdgcn_perm(hiB, loB, 0x07030602u)};
}

// The same 8 levels in natural k order (code 2p, 2p + 1 in dword p).
__device__ __forceinline__ u32x4 nf4_dequant8(uint32_t d)
{
    const u32x4 v = nf4_levels8_kperm(d);
    return u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                 __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
}

}  // namespace q4k
