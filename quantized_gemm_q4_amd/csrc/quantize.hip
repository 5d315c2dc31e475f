// Quantizer kernels for gfx950: group-wise INT4 quantize + pack, per-row INT8
// (per-output-channel weights, per-token activations) and the SmoothQuant
// migration factor.
//
// Built with -ffp-contract=off and IEEE-correct fp32 division and square
// root: these kernels decide integer codes from floating point, and the codes
// must be the same as the round-to-nearest-even formulas give in binary32.
//
// Pages: Core ideas (ai-infra.cypggs.com) §2.2 rounding formulas, §2.3
// granularity, §2.4 migration; Quantization operators guide
// (blog.freezetheflame.cc) §2.1 sym/asym, §2.2 per-channel/per-group, §2.3
// quantize kernel, §5.1 SmoothQuant factor; Quantization notes
// (learn.longtimenohack.com) item (1) group quantization.
#include "q4_internal.hpp"

namespace q4k {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// INT4 quantize + pack. Each lane owns CH chunks of 8 consecutive weights
// (16-byte loads, all issued before any compute); for each chunk the g/8
// lanes of a group reduce min/max (or max|x|) with xor shuffles inside the
// wavefront, so every lane of the group holds the group statistics without a
// broadcast. A block covers CH * 2048 consecutive weights of one row (whole
// groups). Codes leave as one 32-bit store per lane and chunk (8 nibbles,
// even k low), so a wavefront writes 256 contiguous bytes per chunk.
// Zero-points of neighbouring groups meet in LDS to be packed two per byte.
//
// Codes without a division per weight: with x and the fp16 scale sf both
// binary16 values, the exact quotient x / sf is either a tie k + 1/2 or at
// least 2^-16 (relative) away from every tie, while x * rcp(sf) is within a
// few ulp of it; so k = rint(x * rcp(sf)) is rint of the exact quotient
// except at ties, and the remainder r = x - k sf (exact in one fma: both
// terms are multiples of the same power of two and span < 24 bits) is
// exactly +-sf/2 there, where k moves to the even neighbour. The result is
// rint(fl(x / sf)) bit for bit (fl(x / sf) is a tie only when x / sf is).
__device__ __forceinline__ float code_rne(float x, float sf, float inv)
{
    float k = rintf(x * inv);
    const float r = fmaf(-k, sf, x);
    const float half = 0.5f * sf;
    const bool odd = fabsf(k) < 16777216.0f && (((int)k) & 1) != 0;   // |k| >= 2^24 is even
    if (r == half && odd) k += 1.0f;
    if (r == -half && odd) k -= 1.0f;
    return k;
}

template <int LANES, int CH, bool SYM>
__global__ __launch_bounds__(kThreads) void q4_quantize_pack_kernel(
    const uint16_t *__restrict__ W, int64_t K, int G, int chunks_per_row,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros)
{
    constexpr int GPB = kThreads / LANES;   // groups per block and chunk pass
    constexpr int g = LANES * 8;
    __shared__ uint8_t zp_s[GPB * CH];

    const int64_t n = blockIdx.x / chunks_per_row;
    const int c = blockIdx.x % chunks_per_row;
    const int t = threadIdx.x;
    const int gi = t / LANES, li = t % LANES;

    u32x4 raw[CH];
#pragma unroll
    for (int p = 0; p < CH; p++) {
        const int j = (c * CH + p) * GPB + gi;
        raw[p] = u32x4{0u, 0u, 0u, 0u};
        if (j < G) raw[p] = *reinterpret_cast<const u32x4 *>(W + n * K + (int64_t)j * g + li * 8);
    }
#pragma unroll
    for (int p = 0; p < CH; p++) {
        const int j = (c * CH + p) * GPB + gi;
        const bool valid = j < G;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            x[2 * i] = h2f((uint16_t)(raw[p][i] & 0xffffu));
            x[2 * i + 1] = h2f((uint16_t)(raw[p][i] >> 16));
        }
        float lo = 0.0f, hi = 0.0f;   // SYM: hi carries max|x|
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (SYM) {
                hi = fmaxf(hi, fabsf(x[i]));
            } else {
                lo = fminf(lo, x[i]);
                hi = fmaxf(hi, x[i]);
            }
        }
#pragma unroll
        for (int off = LANES / 2; off > 0; off >>= 1) {
            if (!SYM) lo = fminf(lo, __shfl_xor(lo, off));
            hi = fmaxf(hi, __shfl_xor(hi, off));
        }

        const float s32 = SYM ? hi / 7.0f : (hi - lo) / 15.0f;   // IEEE division: rounded to fp16 next
        uint16_t s16 = f2h(s32);
        if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;   // 1.0
        const float sf = h2f(s16);
        const float inv = __builtin_amdgcn_rcpf(sf);
        float zp = 8.0f;
        if (!SYM) zp = fminf(fmaxf(code_rne(-lo, sf, inv), 0.0f), 15.0f);

        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float q = code_rne(x[i], sf, inv);
            if (SYM) {
                q = fminf(fmaxf(q, -8.0f), 7.0f) + 8.0f;
            } else {
                q = fminf(fmaxf(q + zp, 0.0f), 15.0f);
            }
            word |= (uint32_t)q << (4 * i);
        }
        if (valid) {
            const int64_t elem = n * K + (int64_t)j * g + li * 8;
            *reinterpret_cast<uint32_t *>(codes + elem / 2) = word;
            if (li == 0) scales[n * G + j] = s16;
        }
        if (!SYM && li == 0) zp_s[p * GPB + gi] = valid ? (uint8_t)zp : 0;
    }
    if (!SYM) {
        __syncthreads();
        const int Gz = (G + 1) / 2;
        if (t < GPB * CH / 2) {
            const int jz = c * (GPB * CH / 2) + t;
            if (2 * jz < G)
                zeros[n * Gz + jz] = (uint8_t)(zp_s[2 * t] | (zp_s[2 * t + 1] << 4));
        }
    }
}

template <int LANES>
hipError_t launch_q4_g(const uint16_t *W, int64_t N, int64_t K, int sym, uint8_t *codes,
                       uint16_t *scales, uint8_t *zeros, hipStream_t st)
{
    constexpr int GPB = kThreads / LANES;
    constexpr int CH = 2;
    const int G = (int)(K / (LANES * 8));
    const int chunks = (G + GPB * CH - 1) / (GPB * CH);
    const int64_t blocks = N * chunks;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (sym)
        q4_quantize_pack_kernel<LANES, CH, true><<<(unsigned)blocks, kThreads, 0, st>>>(
            W, K, G, chunks, codes, scales, zeros);
    else
        q4_quantize_pack_kernel<LANES, CH, false><<<(unsigned)blocks, kThreads, 0, st>>>(
            W, K, G, chunks, codes, scales, zeros);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row INT8 (Operators guide §2.2 per-channel; the same arithmetic serves
// per-token activations): row values v = x * s (weights, DIV = false) or
// v = x / s (activations, DIV = true), scale = max(max|v|, 1e-8) / 127,
// q = clip(rne(v / scale), -127, 127). One block per row; each lane owns
// 8-element chunks (16-byte loads, 8-byte stores). With CPT > 0 the row's
// values stay in registers between the max pass and the code pass
// (K <= CPT * 2048); CPT == 0 re-reads the row.
__device__ __forceinline__ float block_max(float v, float *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return v;
}

template <bool DIV>
__device__ __forceinline__ void load_row_chunk(const uint16_t *__restrict__ row,
                                               const float *__restrict__ s, int64_t k0,
                                               float v[8])
{
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(row + k0);
    float sv[8];
    if (s) {
        const floatx4 a = *reinterpret_cast<const floatx4 *>(s + k0);
        const floatx4 b = *reinterpret_cast<const floatx4 *>(s + k0 + 4);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            sv[i] = a[i];
            sv[4 + i] = b[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = h2f((uint16_t)(raw[i] & 0xffffu));
        v[2 * i + 1] = h2f((uint16_t)(raw[i] >> 16));
    }
    if (s) {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = DIV ? v[i] / sv[i] : v[i] * sv[i];
    }
}

__device__ __forceinline__ u32x2 q8_codes(const float v[8], float scale)
{
    u32x2 out = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float q = fminf(fmaxf(rintf(v[i] / scale), -127.0f), 127.0f);
        out[i / 4] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (i % 4));
    }
    return out;
}

template <bool DIV, int CPT>
__global__ __launch_bounds__(kThreads) void q8_rows_kernel(const uint16_t *__restrict__ X,
                                                          const float *__restrict__ s,
                                                          int64_t K, int8_t *__restrict__ Q,
                                                          float *__restrict__ scale_out)
{
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const uint16_t *row = X + r * K;
    int8_t *qrow = Q + r * K;
    const int64_t step = (int64_t)kThreads * 8;
    float a = 0.0f;
    if (CPT > 0) {
        float v[CPT > 0 ? CPT : 1][8];
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int64_t k0 = threadIdx.x * 8 + c * step;
            if (k0 < K) {
                load_row_chunk<DIV>(row, s, k0, v[c]);
#pragma unroll
                for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(v[c][i]));
            }
        }
        a = fmaxf(block_max(a, red), 1e-8f);
        const float scale = a / 127.0f;
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int64_t k0 = threadIdx.x * 8 + c * step;
            if (k0 < K) *reinterpret_cast<u32x2 *>(qrow + k0) = q8_codes(v[c], scale);
        }
        if (threadIdx.x == 0) scale_out[r] = scale;
    } else {
        float v[8];
        for (int64_t k0 = threadIdx.x * 8; k0 < K; k0 += step) {
            load_row_chunk<DIV>(row, s, k0, v);
#pragma unroll
            for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(v[i]));
        }
        a = fmaxf(block_max(a, red), 1e-8f);
        const float scale = a / 127.0f;
        for (int64_t k0 = threadIdx.x * 8; k0 < K; k0 += step) {
            load_row_chunk<DIV>(row, s, k0, v);
            *reinterpret_cast<u32x2 *>(qrow + k0) = q8_codes(v, scale);
        }
        if (threadIdx.x == 0) scale_out[r] = scale;
    }
}

template <bool DIV>
hipError_t launch_q8_rows(const uint16_t *X, const float *s, int64_t rows, int64_t K, int8_t *Q,
                          float *scale, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t per = (int64_t)kThreads * 8;
    const int64_t cpt = (K + per - 1) / per;
    const unsigned grid = (unsigned)rows;
    switch (cpt) {
    case 1: q8_rows_kernel<DIV, 1><<<grid, kThreads, 0, st>>>(X, s, K, Q, scale); break;
    case 2: q8_rows_kernel<DIV, 2><<<grid, kThreads, 0, st>>>(X, s, K, Q, scale); break;
    case 3:
    case 4: q8_rows_kernel<DIV, 4><<<grid, kThreads, 0, st>>>(X, s, K, Q, scale); break;
    default: q8_rows_kernel<DIV, 0><<<grid, kThreads, 0, st>>>(X, s, K, Q, scale); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SmoothQuant factor. A block owns 64 input channels: 8 lanes x 8 channels
// across (16-byte loads) by 32 row lanes down; each lane keeps the running
// max|.| of its 8 channels over every 32nd row of Xcal and of W, then the 32
// row lanes meet in LDS. s = ax^a / aw^(1-a), maxima floored at 1e-8.
__global__ __launch_bounds__(kThreads) void smooth_scales_kernel(
    const uint16_t *__restrict__ Xc, int64_t R, const uint16_t *__restrict__ W, int64_t N,
    int64_t K, float alpha, float *__restrict__ s)
{
    __shared__ float mx[32][65];
    __shared__ float mw[32][65];
    const int cl = threadIdx.x % 8;     // 8-channel chunk within the block's 64
    const int rl = threadIdx.x / 8;     // row lane 0..31
    const int64_t k0 = (int64_t)blockIdx.x * 64 + cl * 8;
    float ax[8], aw[8];
#pragma unroll
    for (int i = 0; i < 8; i++) ax[i] = aw[i] = 0.0f;
    if (k0 < K) {
        for (int64_t r = rl; r < R; r += 32) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(Xc + r * K + k0);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                ax[2 * i] = fmaxf(ax[2 * i], fabsf(h2f((uint16_t)(raw[i] & 0xffffu))));
                ax[2 * i + 1] = fmaxf(ax[2 * i + 1], fabsf(h2f((uint16_t)(raw[i] >> 16))));
            }
        }
        for (int64_t r = rl; r < N; r += 32) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(W + r * K + k0);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                aw[2 * i] = fmaxf(aw[2 * i], fabsf(h2f((uint16_t)(raw[i] & 0xffffu))));
                aw[2 * i + 1] = fmaxf(aw[2 * i + 1], fabsf(h2f((uint16_t)(raw[i] >> 16))));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
        mx[rl][cl * 8 + i] = ax[i];
        mw[rl][cl * 8 + i] = aw[i];
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
        float a = 0.0f, b = 0.0f;
        for (int i = 0; i < 32; i++) {
            a = fmaxf(a, mx[i][threadIdx.x]);
            b = fmaxf(b, mw[i][threadIdx.x]);
        }
        a = fmaxf(a, 1e-8f);
        b = fmaxf(b, 1e-8f);
        if (k < K) s[k] = (alpha == 0.5f) ? sqrtf(a) / sqrtf(b)
                                          : powf(a, alpha) / powf(b, 1.0f - alpha);
    }
}

}  // namespace

hipError_t launch_q4_quantize_pack(const uint16_t *W, int64_t N, int64_t K, int g, int sym,
                                   uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                                   hipStream_t st)
{
    switch (g) {
    case 32: return launch_q4_g<4>(W, N, K, sym, codes, scales, zeros, st);
    case 64: return launch_q4_g<8>(W, N, K, sym, codes, scales, zeros, st);
    case 128: return launch_q4_g<16>(W, N, K, sym, codes, scales, zeros, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_q8_weight(const uint16_t *W, const float *s, int64_t N, int64_t K, int8_t *Wq,
                            float *sw, hipStream_t st)
{
    return launch_q8_rows<false>(W, s, N, K, Wq, sw, st);
}

hipError_t launch_q8_act(const uint16_t *X, const float *s, int64_t M, int64_t K, int8_t *Xq,
                         float *sx, hipStream_t st)
{
    return launch_q8_rows<true>(X, s, M, K, Xq, sx, st);
}

hipError_t launch_smooth_scales(const uint16_t *Xcal, int64_t R, const uint16_t *W, int64_t N,
                                int64_t K, float alpha, float *s, hipStream_t st)
{
    const int64_t blocks = (K + 63) / 64;
    if (blocks == 0) return hipSuccess;
    smooth_scales_kernel<<<(unsigned)blocks, kThreads, 0, st>>>(Xcal, R, W, N, K, alpha, s);
    return hipGetLastError();
}

}  // namespace q4k
