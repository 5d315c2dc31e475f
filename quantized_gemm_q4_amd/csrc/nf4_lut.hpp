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

// 8 codes (one dword, code i in nibble i) -> 8 fp16 levels in k order,
// as 4 dwords of pairs (codes 2p, 2p + 1 in dword p)
__device__ __forceinline__ u32x4 nf4_dequant8(uint32_t d)
{
    const uint32_t pos = (d >> 3) & 0x11111111u;                  // 1 where the level is positive
    const uint32_t neg = pos ^ 0x11111111u;
    const uint32_t j = (d ^ (neg * 7u)) & 0x77777777u;            // magnitude index per nibble
    const uint32_t jA = j & 0x0F0F0F0Fu, jB = (j >> 4) & 0x0F0F0F0Fu;   // codes 0,2,4,6 / 1,3,5,7
    const uint32_t loA = __builtin_amdgcn_perm(kNf4Lo1, kNf4Lo0, jA), loB = __builtin_amdgcn_perm(kNf4Lo1, kNf4Lo0, jB);
    const uint32_t hiA = __builtin_amdgcn_perm(kNf4Hi1, kNf4Hi0, jA) | ((neg << 7) & 0x80808080u);
    const uint32_t hiB = __builtin_amdgcn_perm(kNf4Hi1, kNf4Hi0, jB) | ((neg << 3) & 0x80808080u);
    // fp16 of codes 0, 2 | 4, 6 and 1, 3 | 5, 7, then pairs in k order
    const uint32_t a01 = __builtin_amdgcn_perm(hiA, loA, 0x05010400u), a23 = __builtin_amdgcn_perm(hiA, loA, 0x07030602u);
    const uint32_t b01 = __builtin_amdgcn_perm(hiB, loB, 0x05010400u), b23 = __builtin_amdgcn_perm(hiB, loB, 0x07030602u);
    return u32x4{__builtin_amdgcn_perm(b01, a01, 0x05040100u), __builtin_amdgcn_perm(b01, a01, 0x07060302u),
                 __builtin_amdgcn_perm(b23, a23, 0x05040100u), __builtin_amdgcn_perm(b23, a23, 0x07060302u)};
}

}  // namespace q4k
