// NF4 weights on gfx950 (Quantization operators guide §3.4: 16 non-uniform
// levels, the medians of 16 equal-probability intervals of N(0, 1) scaled to
// [-1, 1] and kept in fp16; one fp32 scale per block of 64 weights, the
// block's max |w|; code = index of the level nearest to w / scale; the
// weight is level[code] * scale).
//
// Layout: codes [N, K/2], two 4-bit codes per byte along K (even k in the
// low nibble); scales fp32 [N, K/64].
//
// The decode GEMV dequantizes through a register lookup table: the levels are
// symmetric (level[15 - i] = -level[i]), so a code is a magnitude index j in
// 0..7 and a sign, and v_perm_b32 looks up four bytes at a time in the
// 8-byte tables of the magnitudes' low and high bytes. The exact fp16 levels
// meet x in v_mfma_f32_16x16x32_f16 (every product exact in fp32); each
// 64-block's fp32 partial sum is multiplied by its fp32 scale, so the only
// roundings are fp32 additions and the final fp16 store.
#include <algorithm>
#include <type_traits>

#include "q4_internal.hpp"
#include "nf4_lut.hpp"

namespace q4k {

namespace {

// ---------------------------------------------------------------------------
// Quantizer: a lane owns 8 consecutive weights, 8 lanes one block of 64 (max
// by DPP: quad swaps, then the half-row mirror). w / scale is formed exactly
// (fp64 product with the refined reciprocal, as in the INT8 quantizer:
// fl32(fl64(w * r)) = fl32(w / scale)); the code is the first index of the
// smallest fp32 |x - level| over the 16 levels in ascending order (the
// guide's argmin, ties to the lower index).
__device__ __forceinline__ double nf4_recip64(double b)
{
    double r = __builtin_amdgcn_rcp(b);
    r = fma(fma(-b, r, 1.0), r, r);
    return fma(fma(-b, r, 1.0), r, r);
}

__device__ __forceinline__ float max8(float a)
{
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xF, 0xF, false));
    };
    a = fmaxf(a, dpp(a, std::integral_constant<int, 0xB1>{}));    // quad swap 1 0 3 2
    a = fmaxf(a, dpp(a, std::integral_constant<int, 0x4E>{}));    // quad swap 2 3 0 1
    return fmaxf(a, dpp(a, std::integral_constant<int, 0x141>{}));   // half-row mirror
}

__global__ __launch_bounds__(256) void nf4_quantize_kernel(const uint16_t *__restrict__ W, int64_t N,
                                                           int64_t K, uint8_t *__restrict__ codes,
                                                           float *__restrict__ scales)
{
    const int64_t chunks = K >> 3;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = c < N * chunks;
    const int64_t cc = live ? c : N * chunks - 1;   // idle lanes (whole blocks of 8) redo the last chunk
    const int64_t row = cc / chunks, k0 = (cc % chunks) * 8;
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = h2f((uint16_t)(raw[i] & 0xffffu));
        v[2 * i + 1] = h2f((uint16_t)(raw[i] >> 16));
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    const float a = fmaxf(max8(m), 1e-8f);
    const double r = nf4_recip64((double)a);
    float lv[16];
#pragma unroll
    for (int l = 0; l < 16; l++) lv[l] = h2f(kNf4Levels[l]);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float x = (float)((double)v[i] * r);   // fl32(w / a)
        int best = 0;
        float bd = fabsf(x - lv[0]);
#pragma unroll
        for (int l = 1; l < 16; l++) {
            const float dl = fabsf(x - lv[l]);
            if (dl < bd) {
                bd = dl;
                best = l;
            }
        }
        out |= (uint32_t)best << (4 * i);
    }
    if (live) {
        *reinterpret_cast<uint32_t *>(codes + row * (K >> 1) + (k0 >> 1)) = out;
        if ((threadIdx.x & 7) == 0) scales[row * (K >> 6) + (k0 >> 6)] = a;
    }
}

// ---------------------------------------------------------------------------
// Decode GEMV (M <= 16 rows of X per launch). A block of 8 wavefronts owns 16
// output channels and all of K; wavefront w takes the 128-wide k-blocks
// w, w + 8, w + 16, ..., four at a time: the four k-blocks' code runs (lane
// (r16, q): row r16, k = 32q .. 32q + 31 of the k-block, 16 bytes) and block
// scales are issued together, then computed. X (M rows, natural order) is
// staged in LDS by the whole block. MFMA t of a k-block pairs code dword t
// with X[m][32q + 8t .. + 7]. A k-block spans two 64-blocks with their own
// scales while an MFMA sums over all four lane groups q, so each k-block runs
// two MFMA chains: lanes q < 2 feed the first with their levels and the
// second with zeros, lanes q >= 2 the other way round; the chains' fp32
// results are scaled by the column's two block scales. The wavefronts'
// partial sums meet in LDS.
constexpr int NF4_WAVES = 8, NF4_PF = 4;

__global__ __launch_bounds__(NF4_WAVES * 64) void nf4_gemv_kernel(const uint16_t *__restrict__ X, int M, int N,
                                                                  int K, const uint8_t *__restrict__ codes,
                                                                  const float *__restrict__ scales,
                                                                  uint16_t *__restrict__ Y)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                       // [M][K]
    float *red = reinterpret_cast<float *>(smem + (size_t)M * K * 2);       // [8][4][64]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int n = blockIdx.x * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 6;
    const int KB = K >> 7;

    const int xchunks = (M * K) >> 3;
    for (int c = threadIdx.x; c < xchunks; c += NF4_WAVES * 64)
        *reinterpret_cast<u32x4 *>(xs + c * 8) = *reinterpret_cast<const u32x4 *>(X + (int64_t)c * 8);
    __syncthreads();

    const uint16_t *xrow = xs + (r16 < M ? r16 : M - 1) * K + q * 32;
    const bool first = q < 2;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = wave; kb0 < KB; kb0 += NF4_WAVES * NF4_PF) {
        u32x4 cw[NF4_PF];
        u32x2 sc[NF4_PF];
#pragma unroll
        for (int p = 0; p < NF4_PF; p++) {
            const int kb = kb0 + p * NF4_WAVES;
            const int kc = kb < KB ? kb : KB - 1;   // past the end: a valid k-block, not used
            sc[p] = *reinterpret_cast<const u32x2 *>(scales + (nrow * ks + (uint32_t)kc * 2u));
            cw[p] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)kc * 64u + q * 16u));
        }
#pragma unroll
        for (int p = 0; p < NF4_PF; p++) {
            const int kb = kb0 + p * NF4_WAVES;
            if (kb >= KB) break;
            floatx4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const half8 a = *reinterpret_cast<const half8 *>(xrow + kb * 128 + t * 8);
                const u32x4 w = nf4_dequant8(cw[p][t]);
                const u32x4 z = {0u, 0u, 0u, 0u};
                pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, first ? w : z), pa, 0, 0, 0);
                pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, first ? z : w), pb, 0, 0, 0);
            }
            // (element to a scalar first: a bit_cast of an ext_vector element
            // directly reads element 0 with this compiler)
            const uint32_t s0u = sc[p][0], s1u = sc[p][1];
            const float s0 = __builtin_bit_cast(float, s0u), s1 = __builtin_bit_cast(float, s1u);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(pb[r], s1, fmaf(pa[r], s0, acc[r]));
        }
    }

#pragma unroll
    for (int r = 0; r < 4; r++) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NF4_WAVES; w++) v += red[(w * 4 + r) * 64 + l];
        const int m = 4 * (l >> 4) + r;
        const int nn = blockIdx.x * 16 + (l & 15);
        if (m < M && nn < N) Y[(int64_t)m * N + nn] = f2h(v);
    }
}

}  // namespace

hipError_t launch_nf4_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                               hipStream_t st)
{
    if (N == 0) return hipSuccess;
    const int64_t grid = (N * (K >> 3) + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    nf4_quantize_kernel<<<(unsigned)grid, 256, 0, st>>>(W, N, K, codes, scales);
    return hipGetLastError();
}

// Rows of X in chunks that fit the LDS next to the reduction buffer (at most
// 16 a launch); every block of 8 wavefronts stays resident for N up to 32768.
hipError_t launch_nf4_linear(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                             const float *scales, uint16_t *Y, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (K % 128 != 0 || N * (K / 2) >= (int64_t)0xFFFFFF00) return hipErrorNotSupported;
    // past three passes of the GEMV over the weight, the large-M GEMM with the
    // weight dequantized into LDS once per tile
    if (M > 48) {
        const hipError_t e = launch_nf4_gemm(X, M, N, K, codes, scales, Y, st);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t blocks = (N + 15) / 16;
    if (blocks > 0x7fffffff) return hipErrorNotSupported;
    const size_t red = (size_t)NF4_WAVES * 4 * 64 * 4;
    // up to 16 rows of X per pass, within the 160 KB of LDS; past 64 KB the
    // kernel needs the larger dynamic allocation enabled (once per process)
    constexpr size_t kMaxLds = 160 * 1024;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&nf4_gemv_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)kMaxLds);
    if (attr != hipSuccess) return attr;
    const int64_t rows = std::min<int64_t>(16, (int64_t)((kMaxLds - red) / ((size_t)K * 2)));
    if (rows < 1) return hipErrorNotSupported;
    for (int64_t m0 = 0; m0 < M; m0 += rows) {
        const int m = (int)std::min<int64_t>(rows, M - m0);
        const size_t lds = (size_t)m * K * 2 + red;
        nf4_gemv_kernel<<<(unsigned)blocks, NF4_WAVES * 64, lds, st>>>(X + m0 * K, m, (int)N, (int)K, codes,
                                                                      scales, Y + m0 * N);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4k
