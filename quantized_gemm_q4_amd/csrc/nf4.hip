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

// max over 8 lanes of |w| bit patterns (NaN and the infinities rank above
// every finite value)
__device__ __forceinline__ uint32_t max8_bits(uint32_t a)
{
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false));    // quad swap 1 0 3 2
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false));    // quad swap 2 3 0 1
    return max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x141, 0xF, 0xF, false));   // half-row mirror
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
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __builtin_bit_cast(uint32_t, v[i]) & 0x7fffffffu);
    const uint32_t amax_bits = max8_bits(m);
    // a block holding a NaN or an infinity is flagged: NaN scale, codes 0
    const bool bad = amax_bits >= 0x7f800000u;
    const float a = bad ? 1.0f : fmaxf(__builtin_bit_cast(float, amax_bits), 1e-8f);
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
        *reinterpret_cast<uint32_t *>(codes + row * (K >> 1) + (k0 >> 1)) = bad ? 0u : out;
        if ((threadIdx.x & 7) == 0) scales[row * (K >> 6) + (k0 >> 6)] = bad ? __builtin_nanf("") : a;
    }
}

// ---------------------------------------------------------------------------
// Decode GEMVs (M <= 16 rows of X per launch). A block of 8 wavefronts owns
// 16 output channels and all of K; wavefront w takes the 128-wide k-blocks
// w, w + 8, w + 16, ..., four at a time (a batch): the batch's code runs
// (lane (r16, q): column r16, k = 32q .. 32q + 31 of the k-block, 16 bytes)
// and block scales are issued together, then computed. MFMA t of a k-block
// pairs code dword t with X[.][32q + 8t .. + 7]. X sits in LDS with each run
// of 8 k stored in the order the lookup yields the levels (0, 2, 4, 6, 1, 3,
// 5, 7), so the fragments pair up without a shuffle. A k-block spans two
// 64-blocks (lanes q < 2 and q >= 2) with their own scales while an MFMA sums
// over all four lane groups, so the two halves must land in different
// accumulators. A lane that feeds zeros reads them from a zero run in LDS
// (its k-block stride set to 0). The wavefronts' partial sums meet in LDS.
constexpr int NF4_WAVES = 8, NF4_PF = 4, NF4_ZERO_BYTES = NF4_WAVES * 64;   // zero runs: one of 64 B per wavefront
constexpr size_t NF4_RED_BYTES = (size_t)NF4_WAVES * 4 * 64 * 4;

__device__ __forceinline__ u32x4 nf4_permute_x(u32x4 v)   // x0..x7 -> x0 x2 x4 x6 x1 x3 x5 x7
{
    return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                 __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
}

__device__ __forceinline__ void nf4_load_batch(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                                               uint32_t nrow, uint32_t kh, uint32_t ks, int KB, int kb0, int q,
                                               u32x4 (&cw)[NF4_PF], u32x2 (&sc)[NF4_PF])
{
#pragma unroll
    for (int p = 0; p < NF4_PF; p++) {
        const int kb = kb0 + p * NF4_WAVES;
        const int kc = kb < KB ? kb : KB - 1;   // past the end: a valid k-block, not used
        sc[p] = *reinterpret_cast<const u32x2 *>(scales + (nrow * ks + (uint32_t)kc * 2u));
        cw[p] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)kc * 64u + (uint32_t)q * 16u));
    }
}

__device__ __forceinline__ void nf4_reduce_store(float *red, const floatx4 &acc, bool paired, int M, int N,
                                                 uint16_t *__restrict__ Y)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < 4; r++) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (paired) {
        // output row 2 (l >> 4) + j is the sum of D rows 4 (l >> 4) + 2j, + 2j + 1
        if (threadIdx.x < 128) {
            const int j = threadIdx.x >> 6, l = threadIdx.x & 63;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NF4_WAVES; w++) v += red[(w * 4 + 2 * j) * 64 + l] + red[(w * 4 + 2 * j + 1) * 64 + l];
            const int m = 2 * (l >> 4) + j;
            const int nn = blockIdx.x * 16 + (l & 15);
            if (m < M && nn < N) Y[(int64_t)m * N + nn] = f2h(v);
        }
    } else if (threadIdx.x < 256) {
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NF4_WAVES; w++) v += red[(w * 4 + r) * 64 + l];
        const int m = 4 * (l >> 4) + r;
        const int nn = blockIdx.x * 16 + (l & 15);
        if (m < M && nn < N) Y[(int64_t)m * N + nn] = f2h(v);
    }
}

// M <= 8: A-row 2m + h carries X[m] in the lanes of half h and zeros in the
// others, so D row 2m + h holds half h of row m's sum: one MFMA per 32 k,
// each row scaled by its half's block scale. Each wavefront fetches the X
// runs of its own batch (lane l, load i: row i, k-block kb0 + 8 (l >> 4),
// 16 bytes at 8 (l & 15)) before the batch's codes, so they land first, and
// writes them to an LDS region of its own ([row][k-block of the batch][128
// k], M KB): no block barrier stands between the loads and the compute, and
// K is not bounded by the LDS.
template <int MAXR>   // rows per pass at most (1, 2, 4, 8): the X registers per lane
__global__ __launch_bounds__(NF4_WAVES * 64) void nf4_gemv_paired_kernel(const uint16_t *__restrict__ X, int M,
                                                                         int N, int K,
                                                                         const uint8_t *__restrict__ codes,
                                                                         const float *__restrict__ scales,
                                                                         uint16_t *__restrict__ Y)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned char *xw = smem + (size_t)wave * M * 1024;                          // this wavefront's X runs
    unsigned char *zw = smem + (size_t)NF4_WAVES * M * 1024 + wave * 64;          // and its zero run
    const uint16_t *zs = reinterpret_cast<const uint16_t *>(zw);
    float *red = reinterpret_cast<float *>(smem + (size_t)NF4_WAVES * M * 1024 + NF4_WAVES * 64);
    const int r16 = lane & 15, q = lane >> 4;
    const int n = blockIdx.x * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 6;
    const int KB = K >> 7;

    if (lane < 4) *reinterpret_cast<u32x4 *>(zw + lane * 16) = u32x4{0u, 0u, 0u, 0u};   // read after the barrier below

    const bool live = (r16 >> 1) < M && (r16 & 1) == (q >> 1);
    const uint16_t *fa = live ? reinterpret_cast<const uint16_t *>(xw + (r16 >> 1) * 1024) + q * 32 : zs;
    const int pstride = live ? 128 : 0;   // elements from one k-block of the batch to the next

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = wave; kb0 < KB; kb0 += NF4_WAVES * NF4_PF) {
        const int kx = kb0 + NF4_WAVES * q;   // this lane's X k-block
        u32x4 xv[MAXR];
#pragma unroll
        for (int i = 0; i < MAXR; i++)
            if (i < M && kx < KB)
                xv[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)i * K + (int64_t)kx * 128 + r16 * 8);
        u32x4 cw[NF4_PF];
        u32x2 sc[NF4_PF];
        nf4_load_batch(codes, scales, nrow, kh, ks, KB, kb0, q, cw, sc);
        // the previous batch's LDS reads come before these writes, and the
        // writes before this batch's reads by other lanes of the wavefront:
        // keep the compiler from moving LDS accesses across either point
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < MAXR; i++)
            if (i < M && kx < KB)
                *reinterpret_cast<u32x4 *>(xw + (i * 4 + q) * 256 + r16 * 16) = nf4_permute_x(xv[i]);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < NF4_PF; p++) {
            const int kb = kb0 + p * NF4_WAVES;
            if (kb >= KB) break;
            floatx4 pa = {0.f, 0.f, 0.f, 0.f};
            const uint16_t *f = fa + p * pstride;
#pragma unroll
            for (int t = 0; t < 4; t++)
                pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8 *>(f + t * 8),
                                                            __builtin_bit_cast(half8, nf4_levels8_kperm(cw[p][t])),
                                                            pa, 0, 0, 0);
            // (element to a scalar first: a bit_cast of an ext_vector element
            // directly reads element 0 with this compiler)
            const uint32_t s0u = sc[p][0], s1u = sc[p][1];
            const float s0 = __builtin_bit_cast(float, s0u), s1 = __builtin_bit_cast(float, s1u);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(pa[r], (r & 1) ? s1 : s0, acc[r]);   // D row 4q + r: half r & 1
        }
        asm volatile("" ::: "memory");
    }
    nf4_reduce_store(red, acc, true, M, N, Y);
}

// 9 to 16 rows: two MFMA chains over the same levels, A-row m carrying X[m]
// in half 0's lanes for the first chain and in half 1's for the second. The
// block stages all M rows of X in LDS first.
__global__ __launch_bounds__(NF4_WAVES * 64) void nf4_gemv_kernel(const uint16_t *__restrict__ X, int M, int N,
                                                                  int K, const uint8_t *__restrict__ codes,
                                                                  const float *__restrict__ scales,
                                                                  uint16_t *__restrict__ Y)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                                    // [M][K], k-permuted
    const uint16_t *zs = reinterpret_cast<const uint16_t *>(smem + (size_t)M * K * 2);   // 64 zeros
    float *red = reinterpret_cast<float *>(smem + (size_t)M * K * 2 + NF4_ZERO_BYTES);  // [8][4][64]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int n = blockIdx.x * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 6;
    const int KB = K >> 7;

    const int xchunks = (M * K) >> 3;
    for (int c = threadIdx.x; c < xchunks; c += NF4_WAVES * 64)
        *reinterpret_cast<u32x4 *>(xs + c * 8) = nf4_permute_x(*reinterpret_cast<const u32x4 *>(X + (int64_t)c * 8));
    if (threadIdx.x < NF4_ZERO_BYTES / 16)
        *reinterpret_cast<u32x4 *>(smem + (size_t)M * K * 2 + threadIdx.x * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    const bool half1 = q >= 2;
    const uint16_t *xr = xs + (r16 < M ? r16 : M - 1) * K + q * 32;
    const uint16_t *xa = half1 ? zs : xr, *xb = half1 ? xr : zs;
    const int sa = half1 ? 0 : 128, sb = half1 ? 128 : 0;

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = wave; kb0 < KB; kb0 += NF4_WAVES * NF4_PF) {
        u32x4 cw[NF4_PF];
        u32x2 sc[NF4_PF];
        nf4_load_batch(codes, scales, nrow, kh, ks, KB, kb0, q, cw, sc);
#pragma unroll
        for (int p = 0; p < NF4_PF; p++) {
            const int kb = kb0 + p * NF4_WAVES;
            if (kb >= KB) break;
            floatx4 pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
            const uint16_t *fa = xa + kb * sa, *fb = xb + kb * sb;
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const half8 w = __builtin_bit_cast(half8, nf4_levels8_kperm(cw[p][t]));
                pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8 *>(fa + t * 8), w, pa,
                                                            0, 0, 0);
                pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8 *>(fb + t * 8), w, pb,
                                                            0, 0, 0);
            }
            const uint32_t s0u = sc[p][0], s1u = sc[p][1];
            const float s0 = __builtin_bit_cast(float, s0u), s1 = __builtin_bit_cast(float, s1u);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(pb[r], s1, fmaf(pa[r], s0, acc[r]));
        }
    }
    nf4_reduce_store(red, acc, false, M, N, Y);
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
    // The two-chain form stages all of a pass's rows in LDS (up to 16, within
    // 160 KB); the paired form needs 8 KB per row whatever K is. Past 64 KB
    // the kernels need the larger dynamic allocation enabled (once per process).
    constexpr size_t kMaxLds = 160 * 1024;
    const size_t extra = (size_t)NF4_ZERO_BYTES + NF4_RED_BYTES;
    static const hipError_t attr = [] {
        const void *const fns[] = {reinterpret_cast<const void *>(&nf4_gemv_paired_kernel<8>),
                                   reinterpret_cast<const void *>(&nf4_gemv_kernel)};
        for (const void *f : fns) {
            const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t rows_tc = std::min<int64_t>(16, (int64_t)((kMaxLds - extra) / ((size_t)K * 2)));
    for (int64_t m0 = 0; m0 < M;) {
        const int64_t left = M - m0;
        if (left <= 8 || rows_tc <= 8) {
            const int m = (int)std::min<int64_t>(8, left);
            const size_t lds = (size_t)NF4_WAVES * m * 1024 + extra;
            const dim3 grid((unsigned)blocks), block(NF4_WAVES * 64);
            const uint16_t *Xm = X + m0 * K;
            uint16_t *Ym = Y + m0 * N;
            if (m == 1) nf4_gemv_paired_kernel<1><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym);
            else if (m == 2) nf4_gemv_paired_kernel<2><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym);
            else if (m <= 4) nf4_gemv_paired_kernel<4><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym);
            else nf4_gemv_paired_kernel<8><<<grid, block, lds, st>>>(Xm, m, (int)N, (int)K, codes, scales, Ym);
            m0 += m;
        } else {
            const int m = (int)std::min<int64_t>(rows_tc, left);
            const size_t lds = (size_t)m * K * 2 + extra;
            nf4_gemv_kernel<<<(unsigned)blocks, NF4_WAVES * 64, lds, st>>>(X + m0 * K, m, (int)N, (int)K, codes,
                                                                          scales, Y + m0 * N);
            m0 += m;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4k
