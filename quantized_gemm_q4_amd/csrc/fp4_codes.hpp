// FP4 E2M1 codes on gfx950: the rounding of an fp32 value to its E2M1 code
// (MXFP4 and NVFP4 quantizers) and the register decode of eight E2M1 codes
// to fp16 (NVFP4 weights). E2M1 (Core ideas §2.1; Quantization notes, FP4
// item): sign bit 3, two exponent bits (bias 1), one mantissa bit; the
// values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
#pragma once

#include "q4_internal.hpp"

namespace q4k {

// The E2M1 code of x: the magnitude counted against the format's rounding
// thresholds with ties to the even code -- 0.25 (down), 0.75 (up), 1.25
// (down), 1.75 (up), 2.5 (down), 3.5 (up), 5 (down) -- saturating at 6, and
// the sign bit of x (so -0 keeps its sign).
__device__ __forceinline__ uint32_t e2m1_code(float x)
{
    const float a = fabsf(x);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__builtin_bit_cast(uint32_t, x) >> 28) & 8u);   // sign bit of x
}

// The E2M1 magnitudes are fp16 values with a zero low byte (0x0000, 0x3800,
// 0x3C00, 0x3E00, 0x4000, 0x4200, 0x4400, 0x4600): v_perm_b32 looks up the
// high bytes of four codes at once in this 8-byte table.
constexpr uint32_t kE2m1Hi0 = 0x3E3C3800u, kE2m1Hi1 = 0x46444240u;

// 8 codes (one dword, code i in nibble i) -> their exact fp16 values in k
// order, as 4 dwords of pairs (codes 2p, 2p + 1 in dword p).
__device__ __forceinline__ u32x4 e2m1_dequant8(uint32_t d)
{
    // high bytes of codes 0, 2, 4, 6 (low nibbles; sign bit 3 -> 7) and of
    // codes 1, 3, 5, 7 (high nibbles; the sign is already bit 7)
    const uint32_t hA = __builtin_amdgcn_perm(kE2m1Hi1, kE2m1Hi0, d & 0x07070707u) | ((d << 4) & 0x80808080u);
    const uint32_t hB = __builtin_amdgcn_perm(kE2m1Hi1, kE2m1Hi0, (d >> 4) & 0x07070707u) | (d & 0x80808080u);
    // selector 0x0C yields a zero byte: fp16 (c0, c1) = [0, hA.0, 0, hB.0], ...
    return u32x4{__builtin_amdgcn_perm(hB, hA, 0x040C000Cu), __builtin_amdgcn_perm(hB, hA, 0x050C010Cu),
                 __builtin_amdgcn_perm(hB, hA, 0x060C020Cu), __builtin_amdgcn_perm(hB, hA, 0x070C030Cu)};
}

// An E4M3 scale byte as an fp16 pair (every E4M3 value is an fp16 value).
__device__ __forceinline__ half2v e4m3_half2(uint32_t byte)
{
    const _Float16 h = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
    return half2v{h, h};
}

// 8 NVFP4 codes times their block's E4M3 scale, exact in fp16: an E2M1
// value has at most 2 significant bits and an E4M3 value at most 4, and the
// product lies in [2^-10, 2688], inside fp16's normal range, so the packed
// multiply does not round.
__device__ __forceinline__ u32x4 nvfp4_scaled8(uint32_t d, half2v s2)
{
    const u32x4 v = e2m1_dequant8(d);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const uint32_t w = v[p];   // a scalar first: a bit_cast of a vector element reads element 0 here
        r[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, w) * s2);
    }
    return r;
}

}  // namespace q4k
