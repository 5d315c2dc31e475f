// W4A16 decode GEMV on gfx950: Y[M,N] = X[M,K] * W_hat[N,K]^T for M <= 16 and
// group size 128, with the INT4 weight dequantized in registers (Core ideas,
// ai-infra.cypggs.com, section 2.2: w_hat = (u - zp) * s; Method boundaries,
// llm-glossary.tokens-kit.com, GPTQ section: decode is bound by the weight read).
//
// Arithmetic. v_mfma_f32_16x16x32_f16 takes x in fp16 and 16 (u - zp) as exact
// fp16 integers, so every product is exact in fp32. The fp32 partial sum of one
// 128-wide k-block is multiplied by the fp32 value of the block's group scale
// and added to the fp32 total; the factor 16 is removed at the store. The only
// roundings are fp32 additions and the final fp16 store.
#include <cstdlib>

#include "w4a16_dequant.hpp"

namespace q4k {
namespace {

// Tuning override for the decode GEMV: Q4_GEMV_WAVES=4|8|16 forces the
// wavefronts per block when that configuration is valid for the shape.
int gemv_waves_override()
{
    static const int v = [] {
        const char *e = std::getenv("Q4_GEMV_WAVES");
        const int w = e ? std::atoi(e) : 0;
        return (w == 4 || w == 8 || w == 16) ? w : 0;
    }();
    return v;
}

// ---------------------------------------------------------------------------
// GEMV kernel, small M (decode), g = 128. A block of WAVES wavefronts owns
// 16 output channels and all of K; wavefront w owns exactly KBW k-blocks
// (K = 128 * WAVES * KBW; other shapes take the skinny kernel). Order of
// work, so that compute overlaps the weight stream instead of following it:
//   1. each thread issues its X load (M x K fp16, small, mostly L2 hits),
//      the scales (one vector load) and zero-points (one load) of its
//      k-blocks, then the code loads of all its k-blocks;
//   2. X goes to LDS in the operand k order; the barrier waits only for the
//      X load (loads complete in issue order and X was issued first);
//   3. each k-block is computed as soon as its own codes have landed.
// With every block resident, the whole packed weight is in flight at once.
// A lane whose X row m is >= M feeds row M - 1 instead: MFMA output rows do
// not mix, and rows >= M are never stored. The wavefronts' partial sums meet
// in LDS.
//
// With SM (one X row only) x is replaced by the AWQ-scaled x'' = f2h(x /
// as[k]) as it goes to LDS; the factors are loaded right behind X.
//
// Group sizes 32 and 64 (GS): a lane's 16-byte code run covers the 32 k of
// lane group q, which at g = 32 is a group of its own, so an MFMA step over
// the four lane groups would mix four groups' scales. The four code dwords
// of the four lane groups of a row are transposed first (v_permlane32_swap
// across lane bit 5, v_permlane16_swap across lane bit 4): lane group q then
// holds dword q of every 32-k run of the k-block, MFMA step t takes run t
// (k = 32 t + 8 q .. + 7, one group at g = 32, half of one at g = 64) with
// the X fragments read to match, and each group's exact fp32 partial sum is
// multiplied by that group's scale, as for g = 128.
template <int WAVES, int KBW, bool ASYM, bool ONE_ROW, bool SM = false, int GS = 128, bool PW = false>
__device__ __forceinline__ void gemv_block(const uint16_t *__restrict__ X, int M, int N, int K,
                                           const uint8_t *__restrict__ codes,
                                           const uint16_t *__restrict__ scales,
                                           const uint8_t *__restrict__ zeros, uint16_t *__restrict__ Y,
                                           int blk, const float *__restrict__ as = nullptr)
{
    static_assert(!SM || ONE_ROW, "the fused activation scaling serves one X row");
    static_assert(!PW || !ONE_ROW, "per-wavefront staging of several rows");
    static_assert(KBW == 2 || KBW == 4 || KBW == 8, "vector scale / zero-point loads of 2, 4, 8 groups");
    static_assert(GS == 128 || ((GS == 32 || GS == 64) && KBW <= 4 && !SM), "group sizes 32, 64 up to 4 k-blocks");
    constexpr int GPK = 128 / GS;                            // groups per 128-wide k-block
    constexpr int NS = KBW * GPK;                            // groups of the wavefront's k-blocks
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int kh = K >> 1;                                   // dwords per X row
    uint32_t *xs = reinterpret_cast<uint32_t *>(smem);      // [M][K/2] dwords
    float *red = reinterpret_cast<float *>(xs + M * kh);    // [WAVES][4][64]
    constexpr int kT = WAVES * 64;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int kb0 = wave * KBW;
    const int n = blk * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    const uint32_t G = (uint32_t)K / GS, Gz = (G + 1) >> 1;
    const int xchunks = K >> 3;                              // 16-byte chunks per X row

    // 1. loads: X, scales, zero-points, codes. With one X row each wavefront
    //    fetches just its own k-range of X (no block barrier before the
    //    compute); otherwise the block stages all of X (first row here, one
    //    chunk per thread).
    constexpr int XW = (KBW * 16 + 63) / 64;                 // 16-byte X chunks per lane
    u32x4 xw[XW];
    floatx4 asl[XW], ash[XW];   // SM: the factors of the chunk's 8 columns
    u32x4 x0 = {0u, 0u, 0u, 0u};
    // PW (2 <= M <= 32 / KBW): each wavefront stages the M rows of its own
    // k-range, chunk j = lane + 64 i being row j / (16 KBW), chunk j % (16 KBW)
    // of the k-range; at most 8 chunks per lane
    constexpr int PWC = PW ? 8 : 1;
    u32x4 xp[PWC];
    if (PW) {
#pragma unroll
        for (int i = 0; i < PWC; i++) xp[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < PWC; i++) {
            const int j = lane + 64 * i, m = j / (16 * KBW), c = j % (16 * KBW);
            if (m < M) xp[i] = *reinterpret_cast<const u32x4 *>(X + (m * K + kb0 * 128 + c * 8));
        }
    } else if (ONE_ROW) {
#pragma unroll
        for (int i = 0; i < XW; i++) {
            const int c = lane + 64 * i;
            if (c < KBW * 16) {
                xw[i] = *reinterpret_cast<const u32x4 *>(X + kb0 * 128 + c * 8);
                if (SM) {
                    asl[i] = *reinterpret_cast<const floatx4 *>(as + kb0 * 128 + c * 8);
                    ash[i] = *reinterpret_cast<const floatx4 *>(as + kb0 * 128 + c * 8 + 4);
                }
            }
        }
    } else if ((int)threadIdx.x < xchunks) {
        x0 = *reinterpret_cast<const u32x4 *>(X + threadIdx.x * 8);
    }
    // the scales (NS fp16) and zero-points (NS nibbles) of the wavefront's
    // groups, as whole vector loads (the host checks their alignment)
    uint32_t sraw[NS / 2];
    {
        const uint16_t *sp = scales + (nrow * G + (uint32_t)kb0 * GPK);
        if constexpr (NS >= 8) {
#pragma unroll
            for (int v = 0; v < NS / 8; v++) {
                const u32x4 s8 = reinterpret_cast<const u32x4 *>(sp)[v];
#pragma unroll
                for (int i = 0; i < 4; i++) sraw[4 * v + i] = s8[i];
            }
        } else if constexpr (NS == 4) {
            const u32x2 s4 = *reinterpret_cast<const u32x2 *>(sp);
            sraw[0] = s4[0];
            sraw[1] = s4[1];
        } else {
            sraw[0] = *reinterpret_cast<const uint32_t *>(sp);
        }
    }
    uint64_t zraw = 0x8888888888888888ull;   // symmetric: zp = 8 (no branch, so no early wait)
    if (ASYM) {
        const uint8_t *zp = zeros + (nrow * Gz + ((uint32_t)kb0 * GPK >> 1));
        if constexpr (NS == 16) {
            const u32x2 z = *reinterpret_cast<const u32x2 *>(zp);
            zraw = (uint64_t)z[0] | ((uint64_t)z[1] << 32);
        } else if constexpr (NS == 8) zraw = *reinterpret_cast<const uint32_t *>(zp);
        else if constexpr (NS == 4) zraw = *reinterpret_cast<const uint16_t *>(zp);
        else zraw = *zp;
    }
    u32x4 cw[KBW];
#pragma unroll
    for (int p = 0; p < KBW; p++)
        cw[p] = *reinterpret_cast<const u32x4 *>(codes + (nrow * (uint32_t)kh + (kb0 + p) * 64 + q * 16));

    // 2. X to LDS in the operand order
    if (PW) {
        // only this wavefront reads its k-range of every row: no barrier
#pragma unroll
        for (int i = 0; i < PWC; i++) {
            const int j = lane + 64 * i, m = j / (16 * KBW), c = j % (16 * KBW);
            if (m < M) *reinterpret_cast<u32x4 *>(xs + m * kh + kb0 * 64 + c * 4) = permute_x(xp[i]);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    } else if (ONE_ROW) {
        // only this wavefront reads its k-range: LDS keeps one wavefront's
        // accesses in order, so no barrier
#pragma unroll
        for (int i = 0; i < XW; i++) {
            const int c = lane + 64 * i;
            if (c < KBW * 16)
                *reinterpret_cast<u32x4 *>(xs + kb0 * 64 + c * 4) =
                    permute_x(SM ? awq_div8(xw[i], asl[i], ash[i]) : xw[i]);
        }
        // other lanes of this wavefront read what these lanes wrote: keep
        // the compiler from moving any LDS access across this point (the
        // hardware already runs one wavefront's LDS accesses in order)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    } else {
        if ((int)threadIdx.x < xchunks) *reinterpret_cast<u32x4 *>(xs + threadIdx.x * 4) = permute_x(x0);
        for (int m = 0; m < M; m++) {
            for (int c = threadIdx.x + (m == 0 ? kT : 0); c < xchunks; c += kT) {
                const u32x4 d = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * K + c * 8);
                *reinterpret_cast<u32x4 *>(xs + m * kh + c * 4) = permute_x(d);
            }
        }
        __syncthreads();
    }

    // 3. compute, k-block by k-block. Each group has an accumulator of its
    //    own, so one group's MFMA chain never waits on the previous group's
    //    scaling (a shared accumulator serialises all of them). MFMA step t
    //    reads X chunk 4 q + t of the k-block (g = 128) or 4 t + q (g = 32,
    //    64: the transposed code runs).
    const uint32_t *arow = xs + (r16 < M ? r16 : M - 1) * kh + (GS == 128 ? q * 16 : q * 4) + kb0 * 64;
    floatx4 part[NS];
#pragma unroll
    for (int p = 0; p < KBW; p++) {
        u32x4 w = cw[p];
        if constexpr (GS < 128) {
            const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
            const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
            w = u32x4{s01[0], s01[1], s23[0], s23[1]};
        }
#pragma unroll
        for (int j = 0; j < GPK; j++) part[p * GPK + j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int gi = p * GPK + t * GPK / 4;   // the wavefront's group of this step
            const ZeroConst zc = zero_const((int)(zraw >> (4 * gi)) & 15);
            const half8 a = *reinterpret_cast<const half8 *>(arow + p * 64 + (GS == 128 ? t * 4 : t * 16));
            part[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, dequant8(w[t], zc), part[gi], 0, 0, 0);
        }
    }
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < NS; gi++) {
        const uint32_t sw = sraw[gi >> 1];
        const float sc = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xffffu)));
#pragma unroll
        for (int r = 0; r < 4; r++) acc[r] = fmaf(part[gi][r], sc, acc[r]);
    }

#pragma unroll
    for (int r = 0; r < 4; r++) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; w++) v += red[(w * 4 + r) * 64 + l];
        const int m = 4 * (l >> 4) + r;
        const int nn = blk * 16 + (l & 15);
        if (m < M && nn < N) Y[(int64_t)m * N + nn] = f2h(v * 0.0625f);   // the 1/16 of dequant8
    }
}

template <int WAVES, int KBW, bool ASYM, bool ONE_ROW>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    gemv_block<WAVES, KBW, ASYM, ONE_ROW>(X, M, N, K, codes, scales, zeros, Y, (int)blockIdx.x);
}

// The decode GEMV at group size 32 or 64 (KBW <= 4).
template <int WAVES, int KBW, bool ASYM, bool ONE_ROW, int GS>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_sg_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    gemv_block<WAVES, KBW, ASYM, ONE_ROW, false, GS>(X, M, N, K, codes, scales, zeros, Y, (int)blockIdx.x);
}

// The decode GEMV for 2 <= M <= 32 / KBW rows, each wavefront staging the
// rows of its own k-range (no block barrier before the compute).
template <int WAVES, int KBW, bool ASYM, int GS>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_pw_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    gemv_block<WAVES, KBW, ASYM, false, false, GS, true>(X, M, N, K, codes, scales, zeros, Y, (int)blockIdx.x);
}

// The decode GEMV (one X row) on the AWQ-scaled x'' = f2h(x / awq_s[k]).
template <int WAVES, int KBW, bool ASYM>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_awq_kernel(
    const uint16_t *__restrict__ X, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    const float *__restrict__ awq_s, uint16_t *__restrict__ Y)
{
    gemv_block<WAVES, KBW, ASYM, true, true>(X, 1, N, K, codes, scales, zeros, Y, (int)blockIdx.x,
                                             awq_s);
}

// Several layers that read the same X in one launch: layer i owns blocks
// [first_block_i, first_block_{i+1}); every block runs the GEMV block above
// for its layer. One launch pays the start-up and drain of the weight stream
// once for all the layers.
struct GemvLayer {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint8_t *zeros;
    uint16_t *Y;
    int N, first_block;
};
struct GemvLayers {
    GemvLayer l[kMaxGemvLayers];
    int count;
};

// Layer 0 also comes as leading scalar arguments (the library is built to
// preload the first kernel arguments into scalar registers): its blocks, most
// of the grid in a decode step, start their loads without waiting for a
// kernel-argument load; blocks of the other layers read their layer from L.
template <int WAVES, int KBW, bool ASYM, bool ONE_ROW>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_multi_kernel(
    const uint16_t *__restrict__ X, int M, int K, int first1, const uint8_t *__restrict__ codes0,
    const uint16_t *__restrict__ scales0, const uint8_t *__restrict__ zeros0, uint16_t *__restrict__ Y0, int N0,
    const GemvLayers L)
{
    const int b = (int)blockIdx.x;
    if (b < first1) {
        gemv_block<WAVES, KBW, ASYM, ONE_ROW>(X, M, N0, K, codes0, scales0, zeros0, Y0, b);
        return;
    }
    GemvLayer my = L.l[1];
#pragma unroll
    for (int i = 2; i < kMaxGemvLayers; i++)   // uniform selects, no indexing of the argument
        if (i < L.count && b >= L.l[i].first_block) my = L.l[i];
    gemv_block<WAVES, KBW, ASYM, ONE_ROW>(X, M, my.N, K, my.codes, my.scales, my.zeros, my.Y,
                                          b - my.first_block);
}

// (waves, k-blocks per wavefront) for `blocks` blocks of 16 channels: with
// several X rows the most wavefronts (16, else 8, else 4), with one row 8
// first, that keep every block resident at once (256 CUs x 32 wavefronts), so
// the whole weight is in flight from the start; the k-blocks must divide evenly (2,
// 4 or 8 per wavefront), X must fit in LDS next to the reduction buffer, and
// the scale / zero-point runs of every layer must suit whole vector loads.
bool pick_gemv(int64_t M, int64_t K, int64_t blocks, const uint16_t *const *scales,
               const uint8_t *const *zeros, int count, int &waves_out, int &kbw_out, size_t &lds_out,
               int gs = 128)
{
    const int KB = (int)(K / 128), gpk = 128 / gs;
    const int G = (int)(K / gs), Gz = (G + 1) / 2;
    const int forced = gemv_waves_override();
    // one X row: 8 wavefronts of 4 k-blocks first (with the kernel
    // arguments preloaded, N = 4096: 3.61 against 4.11 us for 16 of 2);
    // several rows: 16 first (the per-wavefront staging takes M * KBW <= 32)
    const int order1[3] = {8, 16, 4}, orderM[3] = {16, 8, 4};
    for (int waves : (M == 1 ? order1 : orderM)) {
        if (forced && waves != forced) continue;
        if (!forced && waves > 4 && blocks * waves > 256 * 32) continue;
        if (KB % waves != 0) continue;
        const int kbw = KB / waves;
        const size_t lds = (size_t)M * K * 2 + (size_t)waves * 4 * 64 * 4;
        if ((kbw != 2 && kbw != 4 && kbw != 8) || (gs < 128 && kbw > 4) || lds > 64 * 1024) continue;
        // a wavefront loads the scales of its ns groups in pieces of up to 16
        // bytes and their zero-points as one load of ns / 2 bytes: every row
        // of both arrays must start on those boundaries
        const int ns = kbw * gpk, ssz = ns * 2 < 16 ? ns * 2 : 16, zsz = ns / 2;
        if ((2 * G) % ssz != 0 || (zsz > 1 && Gz % zsz != 0)) continue;
        bool ok = true;
        for (int i = 0; i < count; i++) {
            if ((reinterpret_cast<uintptr_t>(scales[i]) & (ssz - 1)) != 0) ok = false;
            if (zeros[i] && (reinterpret_cast<uintptr_t>(zeros[i]) & (zsz - 1)) != 0) ok = false;
        }
        if (!ok) continue;
        waves_out = waves;
        kbw_out = kbw;
        lds_out = lds;
        return true;
    }
    return false;
}

}  // namespace

// Launches the GEMV when the shape and the alignment of the scale and
// zero-point arrays suit it; hipErrorNotSupported otherwise (the caller then
// takes another kernel).
// Q4_GEMV_DISPATCH(KERNEL) calls launch(KERNEL<waves, kbw, asym, one_row>).
#define Q4_GEMV_DISPATCH(KERNEL)                                                                  \
    do {                                                                                          \
        auto launch4 = [&](auto k_a1, auto k_a0, auto k_s1, auto k_s0) {                          \
            if (asym) one_row ? launch(k_a1) : launch(k_a0);                                      \
            else one_row ? launch(k_s1) : launch(k_s0);                                           \
        };                                                                                        \
        if (waves == 4 && kbw == 8) Q4_GEMV4(KERNEL, 4, 8);                                       \
        else if (waves == 4 && kbw == 4) Q4_GEMV4(KERNEL, 4, 4);                                  \
        else if (waves == 4) Q4_GEMV4(KERNEL, 4, 2);                                              \
        else if (waves == 8 && kbw == 8) Q4_GEMV4(KERNEL, 8, 8);                                  \
        else if (waves == 8 && kbw == 4) Q4_GEMV4(KERNEL, 8, 4);                                  \
        else if (waves == 8) Q4_GEMV4(KERNEL, 8, 2);                                              \
        else if (kbw == 8) Q4_GEMV4(KERNEL, 16, 8);                                               \
        else if (kbw == 4) Q4_GEMV4(KERNEL, 16, 4);                                               \
        else Q4_GEMV4(KERNEL, 16, 2);                                                             \
    } while (0)
#define Q4_GEMV4(KERNEL, W, B)                                                                    \
    launch4(KERNEL<W, B, true, true>, KERNEL<W, B, true, false>, KERNEL<W, B, false, true>,       \
            KERNEL<W, B, false, false>)

hipError_t launch_w4a16_gemv(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                             const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                             uint16_t *Y, hipStream_t st)
{
    if ((g != 128 && g != 64 && g != 32) || K % 128 != 0 || M > 16 ||
        N * K / 2 >= (int64_t)0xFFFFFF00)   // 32-bit offsets in the kernel
        return hipErrorNotSupported;
    const int m = (int)M, n = (int)N, k = (int)K;
    const int blocks = (n + 15) / 16;
    int waves, kbw;
    size_t lds;
    if (!pick_gemv(M, K, blocks, &scales, &zeros, 1, waves, kbw, lds, g)) return hipErrorNotSupported;
    const bool asym = zeros != nullptr, one_row = m == 1;
    auto launch = [&](auto kernel) {
        kernel<<<blocks, waves * 64, lds, st>>>(X, m, n, k, codes, scales, zeros, Y);
    };
    // several rows that fit 8 staging chunks per lane: per-wavefront staging
    // (Q4_GEMV_PW=0 keeps the block-staged form; read at every call)
    const char *pw_env = std::getenv("Q4_GEMV_PW");
    if (m > 1 && m * kbw <= 32 && !(pw_env && std::atoi(pw_env) == 0)) {
        auto pw2 = [&](auto k_a, auto k_s) { asym ? launch(k_a) : launch(k_s); };
#define Q4_PW(W, B, GS) pw2(w4a16_gemv_pw_kernel<W, B, true, GS>, w4a16_gemv_pw_kernel<W, B, false, GS>)
#define Q4_PW_WB(GS)                                                                              \
    do {                                                                                          \
        if (waves == 4 && kbw == 4) Q4_PW(4, 4, GS);                                              \
        else if (waves == 4) Q4_PW(4, 2, GS);                                                     \
        else if (waves == 8 && kbw == 4) Q4_PW(8, 4, GS);                                         \
        else if (waves == 8) Q4_PW(8, 2, GS);                                                     \
        else if (kbw == 4) Q4_PW(16, 4, GS);                                                      \
        else Q4_PW(16, 2, GS);                                                                    \
    } while (0)
        if (g == 128 && kbw == 8) {
            if (waves == 4) Q4_PW(4, 8, 128);
            else if (waves == 8) Q4_PW(8, 8, 128);
            else Q4_PW(16, 8, 128);
        } else if (g == 128) Q4_PW_WB(128);
        else if (g == 64) Q4_PW_WB(64);   // pick_gemv gives g < 128 at most 4 k-blocks per wavefront
        else Q4_PW_WB(32);
#undef Q4_PW_WB
#undef Q4_PW
        return hipGetLastError();
    }
    if (g == 128) {
        Q4_GEMV_DISPATCH(w4a16_gemv_kernel);
        return hipGetLastError();
    }
    // group sizes 32 and 64: 2 or 4 k-blocks per wavefront
    auto launch4 = [&](auto k_a1, auto k_a0, auto k_s1, auto k_s0) {
        if (asym) one_row ? launch(k_a1) : launch(k_a0);
        else one_row ? launch(k_s1) : launch(k_s0);
    };
#define Q4_SG(W, B, GS)                                                                           \
    launch4(w4a16_gemv_sg_kernel<W, B, true, true, GS>, w4a16_gemv_sg_kernel<W, B, true, false, GS>, \
            w4a16_gemv_sg_kernel<W, B, false, true, GS>, w4a16_gemv_sg_kernel<W, B, false, false, GS>)
#define Q4_SG_W(GS)                                                                               \
    do {                                                                                          \
        if (waves == 4 && kbw == 4) Q4_SG(4, 4, GS);                                              \
        else if (waves == 4) Q4_SG(4, 2, GS);                                                     \
        else if (waves == 8 && kbw == 4) Q4_SG(8, 4, GS);                                         \
        else if (waves == 8) Q4_SG(8, 2, GS);                                                     \
        else if (kbw == 4) Q4_SG(16, 4, GS);                                                      \
        else Q4_SG(16, 2, GS);                                                                    \
    } while (0)
    if (g == 64) Q4_SG_W(64);
    else Q4_SG_W(32);
#undef Q4_SG_W
#undef Q4_SG
    return hipGetLastError();
}

hipError_t launch_w4a16_gemv_multi(const uint16_t *X, int64_t M, int64_t K, int g,
                                   const GemvLayerDesc *layers, int count, hipStream_t st)
{
    if (g != 128 || M > 16 || count < 1 || count > kMaxGemvLayers) return hipErrorNotSupported;
    const bool asym = layers[0].zeros != nullptr;
    GemvLayers L{};
    const uint16_t *sc[kMaxGemvLayers];
    const uint8_t *zp[kMaxGemvLayers];
    int64_t blocks = 0;
    for (int i = 0; i < count; i++) {
        const GemvLayerDesc &d = layers[i];
        if ((d.zeros != nullptr) != asym || d.N * K / 2 >= (int64_t)0xFFFFFF00)
            return hipErrorNotSupported;
        L.l[i] = GemvLayer{d.codes, d.scales, d.zeros, d.Y, (int)d.N, (int)blocks};
        sc[i] = d.scales;
        zp[i] = d.zeros;
        blocks += (d.N + 15) / 16;
    }
    L.count = count;
    if (blocks == 0) return hipSuccess;
    int waves, kbw;
    size_t lds;
    if (!pick_gemv(M, K, blocks, sc, zp, count, waves, kbw, lds)) return hipErrorNotSupported;
    const int m = (int)M, k = (int)K;
    const bool one_row = m == 1;
    const int first1 = count > 1 ? L.l[1].first_block : (int)blocks;
    const GemvLayer &l0 = L.l[0];
    auto launch = [&](auto kernel) {
        kernel<<<(int)blocks, waves * 64, lds, st>>>(X, m, k, first1, l0.codes, l0.scales, l0.zeros, l0.Y, l0.N, L);
    };
    Q4_GEMV_DISPATCH(w4a16_gemv_multi_kernel);
    return hipGetLastError();
}
hipError_t launch_w4a16_gemv_awq(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                                 const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                                 const float *awq_s, uint16_t *Y, hipStream_t st)
{
    if (g != 128 || M != 1 || N * K / 2 >= (int64_t)0xFFFFFF00) return hipErrorNotSupported;
    const int n = (int)N, k = (int)K;
    const int blocks = (n + 15) / 16;
    int waves, kbw;
    size_t lds;
    if (!pick_gemv(M, K, blocks, &scales, &zeros, 1, waves, kbw, lds)) return hipErrorNotSupported;
    auto launch = [&](auto kernel) {
        kernel<<<blocks, waves * 64, lds, st>>>(X, n, k, codes, scales, zeros, awq_s, Y);
    };
#define Q4_AWQ(W, B)                                                                              \
    (zeros ? launch(w4a16_gemv_awq_kernel<W, B, true>) : launch(w4a16_gemv_awq_kernel<W, B, false>))
    if (waves == 4 && kbw == 8) Q4_AWQ(4, 8);
    else if (waves == 4 && kbw == 4) Q4_AWQ(4, 4);
    else if (waves == 4) Q4_AWQ(4, 2);
    else if (waves == 8 && kbw == 8) Q4_AWQ(8, 8);
    else if (waves == 8 && kbw == 4) Q4_AWQ(8, 4);
    else if (waves == 8) Q4_AWQ(8, 2);
    else if (kbw == 8) Q4_AWQ(16, 8);
    else if (kbw == 4) Q4_AWQ(16, 4);
    else Q4_AWQ(16, 2);
#undef Q4_AWQ
    return hipGetLastError();
}
#undef Q4_GEMV4
#undef Q4_GEMV_DISPATCH

}  // namespace q4k
