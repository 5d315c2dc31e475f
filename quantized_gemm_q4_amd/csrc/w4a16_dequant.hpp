// Exact INT4 unpack helpers shared by the W4A16 kernels (gfx950).
//
// Operand layout. In a 16x16x32 MFMA lane l feeds row (l % 16) of A and column
// (l % 16) of B with 8 k-values each; A and B see the same k order, so the
// product does not depend on which k sits where. The unpack below picks the
// order that makes it cheap: lane group q = l / 16 owns the 32 consecutive k
// of a 128-wide k-block starting at 32q (one 16-byte load of codes), and
// MFMA step t takes the 8 nibbles of the lane's dword t. Masks of the form
// 0x000F000F lift nibbles i and i+4 into the two fp16 halves of a register at
// once, so the B operand holds k offsets (0,4,1,5,2,6,3,7); the X operand is
// permuted the same way (permute_x).
#pragma once

#include "q4_internal.hpp"

namespace q4k {

// Dequantize the 8 nibbles of one code dword (nib_i at bits 4i, k offset i)
// into 16 * (nib - zp) as exact fp16 integers, in the operand k order
// (0,4,1,5,2,6,3,7). OR-ing a nibble into the mantissa of fp16 1024.0
// (0x6400) makes 1024 + nib when the nibble sits at bits 0-3 of a half and
// 1024 + 16 * nib when it sits at bits 4-7; both are exact. So one mask
// serves nibbles i and i+4 at bit 0 and another nibbles i+1 and i+5 at bit 4;
// only one shift (by 8) is needed per dword. The bit-0 pairs are brought to
// the same 16x scale with one fused multiply-add, the bit-4 pairs with one
// subtraction: 16 (1024 + n) - (16384 + 16 zp) and (1024 + 16 n) - (1024 + 16
// zp) are exact. The caller folds the factor 1/16 into the fp32 scale.
struct ZeroConst {
    uint32_t lo;   // fp16 pair -(16384 + 16 zp)
    uint32_t hi;   // fp16 pair   1024 + 16 zp
};

__device__ __forceinline__ ZeroConst zero_const(int zp)
{
    return ZeroConst{(uint32_t)(0xF400 + zp) * 0x10001u, (uint32_t)(0x6400 + 16 * zp) * 0x10001u};
}

// (w & mask) | magic in one v_and_or_b32. The backend does not fuse the two
// when both constants are literals; this is plain ALU, no memory operand.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

__device__ __forceinline__ half8 dequant8(uint32_t w, ZeroConst z)
{
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, magic = 0x64006400u;
    const half2v sixteen = {(_Float16)16.0f, (_Float16)16.0f};
    const half2v zl = __builtin_bit_cast(half2v, z.lo);
    const half2v zh = __builtin_bit_cast(half2v, z.hi);
    const uint32_t w8 = w >> 8;
    const half2v p0 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, and_or(w, lo, magic)), sixteen, zl);
    const half2v p1 = __builtin_bit_cast(half2v, and_or(w, hi, magic)) - zh;
    const half2v p2 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, and_or(w8, lo, magic)), sixteen, zl);
    const half2v p3 = __builtin_bit_cast(half2v, and_or(w8, hi, magic)) - zh;
    const u32x4 r = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                     __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    return __builtin_bit_cast(half8, r);
}

// fp32 value of a group scale with the 1/16 of dequant8 folded in (exact).
__device__ __forceinline__ float scale16(uint16_t s) { return h2f(s) * 0.0625f; }

// Natural-order fp16 x0..x7 (four dwords) -> (x0,x4,x1,x5,x2,x6,x3,x7).
__device__ __forceinline__ u32x4 permute_x(u32x4 d)
{
    u32x4 r;
    r[0] = (d[0] & 0xffffu) | (d[2] << 16);
    r[1] = (d[0] >> 16) | (d[2] & 0xffff0000u);
    r[2] = (d[1] & 0xffffu) | (d[3] << 16);
    r[3] = (d[1] >> 16) | (d[3] & 0xffff0000u);
    return r;
}

__device__ __forceinline__ int group_zp(const uint8_t *__restrict__ zeros, int64_t n, int Gz,
                                        int grp)
{
    if (!zeros) return 8;
    return (zeros[n * Gz + (grp >> 1)] >> ((grp & 1) * 4)) & 15;
}

}  // namespace q4k
