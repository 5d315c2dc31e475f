// NVFP4 weights on gfx950 (Quantization notes, FP4 item: FP4 E2M1 values with
// one FP8 E4M3 scale per block of 16, 4 + 8/16 = 4.5 bits per weight; its
// NVFP4-style sketch: scale = E4M3(amax / 6), code = the E2M1 value of
// w / scale, clipped to +-6).
//
// Layout: codes [N, K/2], two E2M1 codes per byte along K (even k in the low
// nibble); scales [N, K/16] E4M3 bytes.
//
// gfx950's block-scaled matrix cores take E8M0 scales on blocks of 32, not
// E4M3 scales on blocks of 16, so these weights meet fp16 X on the fp16
// matrix cores: e2m1 * e4m3 is exact in fp16 (at most 6 significant bits, in
// [2^-10, 2688]), so the block scale is folded into the operand without a
// rounding, and the products and fp32 sums are the W4A16 kernels' own.
#include <algorithm>
#include <type_traits>

#include "fp4_codes.hpp"
#include "q4_internal.hpp"
#include "row_codes.hpp"

namespace q4k {

namespace {

// ---------------------------------------------------------------------------
// Quantizer: a lane owns 8 consecutive weights, two neighbouring lanes one
// block of 16 (max by one DPP swap). fl32(amax / 6) comes from the fp64
// product with the nearest double to 1/6 (within 2^-53 of it; an fp16-valued
// amax over the binary32 6 stays 2^-49 away from any binary32 midpoint, so
// the product rounds as the quotient does), clamped to 448 and converted to
// E4M3 by v_cvt_pk_fp8_f32 (nearest, ties to even). With a nonzero scale,
// w / scale is formed as fl32(fl64(w * r)) with r the refined fp64
// reciprocal of the scale (the same argument), and e2m1_code rounds it.
__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(const uint16_t *__restrict__ W, int64_t N,
                                                             int64_t K, uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales)
{
    const int64_t chunks = K >> 3;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = c < N * chunks;
    const int64_t cc = live ? c : N * chunks - 1;   // idle lanes (whole pairs) redo the last chunk
    const int64_t row = cc / chunks, k0 = (cc % chunks) * 8;
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = h2f((uint16_t)(raw[i] & 0xffffu));
        v[2 * i + 1] = h2f((uint16_t)(raw[i] >> 16));
    }
    // max of |w| bit patterns (NaN and the infinities rank above every finite
    // value); the two lanes of a block are neighbours (chunks per row is even)
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __builtin_bit_cast(uint32_t, v[i]) & 0x7fffffffu);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    // a block holding a NaN or an infinity is flagged: scale byte 0x7f
    // (E4M3's NaN), codes 0
    const bool bad = m >= 0x7f800000u;
    const float amax = bad ? 0.0f : __builtin_bit_cast(float, m);
    const float q = (float)((double)amax * (1.0 / 6.0));   // fl32(amax / 6)
    const uint32_t sc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(q, 448.0f), 0.0f, 0, false) & 0xFFu;
    const float scale = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
    uint32_t out = 0;
    if (scale > 0.0f) {
        const double r = recip64((double)scale);
#pragma unroll
        for (int i = 0; i < 8; i++) out |= e2m1_code((float)((double)v[i] * r)) << (4 * i);
    }
    if (live) {
        *reinterpret_cast<uint32_t *>(codes + row * (K >> 1) + (k0 >> 1)) = out;
        if ((threadIdx.x & 1) == 0) scales[row * (K >> 4) + (k0 >> 4)] = bad ? (uint8_t)0x7f : (uint8_t)sc;
    }
}

// ---------------------------------------------------------------------------
// Decode GEMV (M <= 16 rows of X per pass). A block of 8 wavefronts owns 16
// output channels and all of K; wavefront w takes the 128-wide k-blocks in
// batches of four consecutive ones (4w .. 4w + 3, then 32 further on, ...), so
// a batch's 32 scale bytes of a row are one window of two 16-byte loads. Lane (r16, q) holds column
// r16's code run for k = 32q .. 32q + 31 of a k-block (16 bytes, two blocks
// of 16) and those two blocks' scale bytes; MFMA t pairs code dword t (scaled
// by block t / 2) with X[r16][32q + 8t .. + 7]. Each wavefront fetches the X
// runs of its own batch (lane l, load i: row i, k-block kb0 + (l >> 4),
// 16 bytes at 8 (l & 15)) before its codes, so they land first, and writes
// them to an LDS region of its own ([row][k-block of the batch][128 k],
// M KB): no block barrier stands between the loads and the compute. A-rows
// past M read a zero run. The wavefronts' partial sums meet in LDS.
constexpr int NV_WAVES = 8, NV_PF = 4, NV_ZERO_BYTES = NV_WAVES * 64;
constexpr size_t NV_RED_BYTES = (size_t)NV_WAVES * 4 * 64 * 4;

template <int MAXR>   // rows per pass at most (1, 2, 4, 8, 16): the X registers per lane
__global__ __launch_bounds__(NV_WAVES * 64) void nvfp4_gemv_kernel(const uint16_t *__restrict__ X, int M, int N,
                                                                   int K, const uint8_t *__restrict__ codes,
                                                                   const uint8_t *__restrict__ scales,
                                                                   uint16_t *__restrict__ Y, int vsc)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned char *xw = smem + (size_t)wave * M * 1024;                       // this wavefront's X runs
    unsigned char *zw = smem + (size_t)NV_WAVES * M * 1024 + wave * 64;       // and its zero run
    float *red = reinterpret_cast<float *>(smem + (size_t)NV_WAVES * M * 1024 + NV_ZERO_BYTES);
    const int r16 = lane & 15, q = lane >> 4;
    const int n = blockIdx.x * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 4;
    const int KB = K >> 7;

    if (lane < 4) *reinterpret_cast<u32x4 *>(zw + lane * 16) = u32x4{0u, 0u, 0u, 0u};   // read after the barrier below

    const bool live = r16 < M;
    const uint16_t *fa = live ? reinterpret_cast<const uint16_t *>(xw + r16 * 1024) + q * 32
                              : reinterpret_cast<const uint16_t *>(zw);
    const int pstride = live ? 128 : 0;   // elements from one k-block of the batch to the next

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = NV_PF * wave; kb0 < KB; kb0 += NV_WAVES * NV_PF) {
        const int kx = kb0 + q;   // this lane's X k-block
        u32x4 xv[MAXR];
#pragma unroll
        for (int i = 0; i < MAXR; i++)
            if (i < M && kx < KB)
                xv[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)i * K + (int64_t)kx * 128 + r16 * 8);
        u32x4 cw[NV_PF];
        uint32_t sc[NV_PF];
        // the batch's 4 k-blocks are consecutive: their 32 scale bytes of the
        // row are one window, two 16-byte loads (vsc: the host found the
        // window aligned); otherwise a 2-byte load per k-block
        const bool win = vsc && kb0 + NV_PF <= KB;
        u32x4 sw0 = {0u, 0u, 0u, 0u}, sw1 = {0u, 0u, 0u, 0u};
        if (win) {
            const uint8_t *sp = scales + (nrow * ks + (uint32_t)kb0 * 8u);
            sw0 = *reinterpret_cast<const u32x4 *>(sp);
            sw1 = *reinterpret_cast<const u32x4 *>(sp + 16);
        }
#pragma unroll
        for (int p = 0; p < NV_PF; p++) {
            const int kb = kb0 + p;
            const int kc = kb < KB ? kb : KB - 1;   // past the end: a valid k-block, not used
            if (!win)
                sc[p] = *reinterpret_cast<const uint16_t *>(scales + (nrow * ks + (uint32_t)kc * 8u + (uint32_t)q * 2u));
            cw[p] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)kc * 64u + (uint32_t)q * 16u));
        }
        if (win) {
            // byte 8 p + 2 q of the window: dword 2 p + q / 2, half q % 2
#pragma unroll
            for (int p = 0; p < NV_PF; p++) {
                const u32x4 &w4 = p < 2 ? sw0 : sw1;
                const uint32_t lo = w4[(2 * p) & 3], hi = w4[(2 * p + 1) & 3];
                sc[p] = ((q & 2) ? hi : lo) >> ((q & 1) * 16) & 0xFFFFu;
            }
        }
        // the previous batch's LDS reads come before these writes, and the
        // writes before this batch's reads by other lanes of the wavefront:
        // keep the compiler from moving LDS accesses across either point
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < MAXR; i++)
            if (i < M && kx < KB) *reinterpret_cast<u32x4 *>(xw + (i * 4 + q) * 256 + r16 * 16) = xv[i];
        asm volatile("" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < NV_PF; p++) {
            const int kb = kb0 + p;
            if (kb >= KB) break;
            const half2v s0 = e4m3_half2(sc[p] & 0xFFu), s1 = e4m3_half2(sc[p] >> 8);
            const uint16_t *f = fa + p * pstride;
#pragma unroll
            for (int t = 0; t < 4; t++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8 *>(f + t * 8),
                                                             __builtin_bit_cast(half8, nvfp4_scaled8(cw[p][t], t < 2 ? s0 : s1)),
                                                             acc, 0, 0, 0);
        }
        asm volatile("" ::: "memory");
    }

#pragma unroll
    for (int r = 0; r < 4; r++) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NV_WAVES; w++) v += red[(w * 4 + r) * 64 + l];
        const int m = 4 * (l >> 4) + r;
        const int nn = blockIdx.x * 16 + (l & 15);
        if (m < M && nn < N) Y[(int64_t)m * N + nn] = f2h(v);
    }
}

}  // namespace

hipError_t launch_nvfp4_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scales,
                                 hipStream_t st)
{
    if (N == 0) return hipSuccess;
    const int64_t threads = N * (K >> 3);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorNotSupported;
    nvfp4_quantize_kernel<<<(unsigned)blocks, 256, 0, st>>>(W, N, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_nvfp4_linear(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                               const uint8_t *scales, uint16_t *Y, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (K % 128 != 0 || N * (K / 2) >= (int64_t)0xFFFFFF00) return hipErrorNotSupported;
    // past three passes of the GEMV over the weight, the large-M GEMM with the
    // weight dequantized into LDS once per tile
    if (M > 48) {
        const hipError_t e = launch_nvfp4_gemm(X, M, N, K, codes, scales, Y, st);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t blocks = (N + 15) / 16;
    if (blocks > 0x7fffffff) return hipErrorNotSupported;
    // 1 KB of X per row per wavefront; past 64 KB the kernel needs the larger
    // dynamic allocation enabled (once per process)
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&nvfp4_gemv_kernel<16>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    // the scale windows of a wavefront's batches are 16-byte aligned when
    // every row starts on 16 bytes (K / 16 a multiple of 16) and so does the array
    const int vsc = (K % 256 == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) ? 1 : 0;
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int m = (int)std::min<int64_t>(16, M - m0);
        const size_t lds = (size_t)NV_WAVES * m * 1024 + NV_ZERO_BYTES + NV_RED_BYTES;
        const dim3 grid((unsigned)blocks), block(NV_WAVES * 64);
        const uint16_t *Xm = X + m0 * K;
        uint16_t *Ym = Y + m0 * N;
        if (m == 1) nvfp4_gemv_kernel<1><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym, vsc);
        else if (m == 2) nvfp4_gemv_kernel<2><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym, vsc);
        else if (m <= 4) nvfp4_gemv_kernel<4><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym, vsc);
        else if (m <= 8) nvfp4_gemv_kernel<8><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym, vsc);
        else nvfp4_gemv_kernel<16><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym, vsc);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4k
