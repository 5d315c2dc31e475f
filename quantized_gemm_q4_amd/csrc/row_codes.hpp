// Per-row INT8 / FP8 E4M3 codes shared by the row quantizers and the decode
// GEMVs that quantize their activations themselves (gfx950).
#pragma once

#include "q4_internal.hpp"

namespace q4k {

// Quotients without a division. For binary32 (or binary16-valued) a and a
// binary32 b the exact quotient a / b never lies on the midpoint between two
// binary32 neighbours, and when it does not it is at least 2^-49 (relative)
// away from one: with a = A 2^ea (A < 2^24) and a midpoint m (25 significant
// bits), a - m b is a nonzero multiple of 2^(ea - 25), so at least 2^-49 of
// a. So a product a * r in fp64 with r within 2^-50 of 1 / b (relative; the
// fp64 rounding of the product adds 2^-53) rounds to the same binary32 value
// as a / b:
// fl32(fl64(a * r)) = fl32(a / b). r is the hardware's fp64 reciprocal
// refined by two Newton steps (each squares the relative error; rounding
// keeps it near 2^-53). b must be finite and nonzero.
__device__ __forceinline__ double recip64(double b)
{
    double r = __builtin_amdgcn_rcp(b);
    r = fma(fma(-b, r, 1.0), r, r);
    return fma(fma(-b, r, 1.0), r, r);
}

// Row formats: INT8 codes rint(v / scale) clipped to +-127, or FP8 E4M3
// codes of v / scale (the nearest E4M3 value, ties to even, sign kept on
// zero; the hardware conversion v_cvt_pk_fp8_f32 rounds to nearest even and
// the quotient is clamped to +-448 first, so nothing saturates in it). The
// scale is max |v| / 127 or max |v| / 448 (Quantization operators guide
// §2.1, §4.2).
template <bool FP8> constexpr float kRowMax = FP8 ? 448.0f : 127.0f;

// four quotients -> four code bytes (quotient i in byte i)
template <bool FP8>
__device__ __forceinline__ uint32_t row_codes4(float q0, float q1, float q2, float q3)
{
    if constexpr (FP8) {
        auto c = [](float q) { return fminf(fmaxf(q, -448.0f), 448.0f); };
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(q0), c(q1), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c(q2), c(q3), w, true);
        return (uint32_t)w;
    } else {
        // clamp to [-127, 127] (integer bounds, so clamping before rounding
        // is the same as after), then 1.5 * 2^23 + q rounds q to the nearest
        // integer, ties to even, and leaves it (two's complement) in the low
        // byte of the sum's bits; three byte permutes pack the four codes
        auto c = [](float q) {
            return __builtin_bit_cast(uint32_t, fminf(fmaxf(q, -127.0f), 127.0f) + 12582912.0f);
        };
        const uint32_t p01 = __builtin_amdgcn_perm(c(q1), c(q0), 0x0c0c0400u);
        const uint32_t p23 = __builtin_amdgcn_perm(c(q3), c(q2), 0x0c0c0400u);
        return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    }
}

// ---------------------------------------------------------------------------
// The per-token quantizer inside a 512-thread decode block (M * K <= 16384,
// K a multiple of 8): thread t owns the 8-element chunks t, t + 512, ... of
// the row-major X. fused_load_x issues the chunks' loads (and their smoothing
// factors); the caller issues its weight loads next, so its weight bytes are
// on the way while fused_quantize_x forms x' = x / s, the row maxima (LDS
// max on the float bit patterns, which order as the values for |x'|), the
// scales max(amax, 1e-8) / 127 (or / 448) by IEEE division and the codes
// rint(fl32(x' / scale)) (or the nearest E4M3) into xq [M][K] in LDS -- the
// row quantizer's arithmetic, so codes and scales are bit for bit its. Block
// 0 also writes them to ws_codes / ws_scale. Ends with a block barrier.
constexpr int kFusedMaxMK = 16384;
constexpr int kFusedChunks = kFusedMaxMK / 8 / 512;

struct FusedX {
    u32x4 xr[kFusedChunks];
    floatx4 slo[kFusedChunks], shi[kFusedChunks];
};

template <bool HAS_S>
__device__ __forceinline__ void fused_load_x(FusedX &f, const uint16_t *__restrict__ X,
                                             const float *__restrict__ s, int nchunks, int K)
{
#pragma unroll
    for (int i = 0; i < kFusedChunks; i++) {
        const int c = (int)threadIdx.x + 512 * i;
        const int cc = c < nchunks ? c : nchunks - 1;
        f.xr[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)cc * 8);
        if (HAS_S) {
            const int k = (cc * 8) % K;
            f.slo[i] = *reinterpret_cast<const floatx4 *>(s + k);
            f.shi[i] = *reinterpret_cast<const floatx4 *>(s + k + 4);
        }
    }
}

template <bool FP8, bool HAS_S>
__device__ __forceinline__ void fused_quantize_x(const FusedX &f, int nchunks, int M, int K,
                                                 uint8_t *xq, uint32_t *rmax, float *rscale,
                                                 uint8_t *__restrict__ ws_codes,
                                                 float *__restrict__ ws_scale)
{
    const int tid = (int)threadIdx.x;
    if (tid < 16) rmax[tid] = 0u;
    __syncthreads();
    float v[kFusedChunks][8];
#pragma unroll
    for (int i = 0; i < kFusedChunks; i++) {
        const int c = tid + 512 * i;
        uint32_t a = 0u;   // max of |v| bit patterns: NaN and the infinities rank above every finite value
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t d = f.xr[i][e >> 1];
            const float x = h2f((uint16_t)((e & 1) ? (d >> 16) : (d & 0xffffu)));
            if (HAS_S) {
                const float sv = e < 4 ? f.slo[i][e] : f.shi[i][e - 4];
                v[i][e] = (float)((double)x * recip64((double)sv));   // fl32(x / s)
            } else {
                v[i][e] = x;
            }
            a = max(a, __builtin_bit_cast(uint32_t, v[i][e]) & 0x7fffffffu);
        }
        if (c < nchunks) atomicMax(&rmax[(c * 8) / K], a);
    }
    __syncthreads();
    // a row holding a NaN or an infinity is flagged: NaN scale, codes 0
    if (tid < M) {
        const bool bad = rmax[tid] >= 0x7f800000u;
        const float a = fmaxf(__builtin_bit_cast(float, rmax[tid]), 1e-8f);
        const float sc = bad ? __builtin_nanf("") : a / kRowMax<FP8>;
        rscale[tid] = sc;
        if (blockIdx.x == 0) ws_scale[tid] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kFusedChunks; i++) {
        const int c = tid + 512 * i;
        if (c < nchunks) {
            const float sr = rscale[(c * 8) / K];
            const bool bad = sr != sr;
            const double rs = recip64((double)(bad ? 1.0f : sr));
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; e++) q[e] = (float)((double)v[i][e] * rs);
            u32x2 out = {row_codes4<FP8>(q[0], q[1], q[2], q[3]), row_codes4<FP8>(q[4], q[5], q[6], q[7])};
            if (bad) out = u32x2{0u, 0u};
            *reinterpret_cast<u32x2 *>(xq + c * 8) = out;
            if (blockIdx.x == 0) *reinterpret_cast<u32x2 *>(ws_codes + (int64_t)c * 8) = out;
        }
    }
    __syncthreads();
}

}  // namespace q4k
