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
#include <type_traits>

#include "q4_internal.hpp"
#include "row_codes.hpp"

namespace q4k {
namespace {

constexpr int kThreads = 256;

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// |v| as a binary32 bit pattern: these order as the magnitudes, and NaN and
// the infinities (0x7f800000 and above) rank above every finite value, so an
// integer maximum over them finds a non-finite value (fmaxf skips NaN)
__device__ __forceinline__ uint32_t abs_bits(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7fffffffu; }
constexpr uint32_t kNonFinite = 0x7f800000u;

// ---------------------------------------------------------------------------
// INT4 quantize + pack. Each lane owns 16 consecutive weights of one group
// (two 16-byte loads); the g/16 lanes of a group (2, 4 or 8, inside one
// half-row of 8 lanes) reduce the group's minimum and maximum (or max |x|)
// with DPP lane exchanges, so every lane holds the group statistics without
// a broadcast. A block covers 4096 consecutive weights of one row (whole
// groups). Minimum and maximum are exact in any precision, so they are taken
// on packed fp16 pairs and the exchanges move (min, -max) together in one
// register.
//
// Codes without a division per weight: with x and the fp16 scale sf both
// binary16 values, the exact quotient x / sf is either a tie k + 1/2 or at
// least 2^-12 (relative) away from every tie, while x * rcp(sf) is within a
// few ulp of it. One fma t = x * rcp(sf) + (1.5 * 2^23 + zp) therefore
// rounds to 1.5 * 2^23 + zp + rint(x / sf) except at ties (adding the
// integer zp cannot move a value that is not a tie across a rounding
// boundary), and a med3 clamps t to [1.5 * 2^23, 1.5 * 2^23 + 15], whose low
// four bits are then the code. Ties are found exactly: the remainder
// r = x - k sf (one fma, exact: both terms are multiples of the same power of
// two and span < 24 bits) is +-sf / 2 there, and k then moves to its even
// neighbour. Ties are rare (a few weights in 10^4 on Gaussian weights), so
// the fix-up runs only in wavefronts that have one. The result is
// clamp(rint(fl(x / sf)) + zp, 0, 15) bit for bit (fl(x / sf) is a tie only
// when x / sf is).

// Lane exchange for the group reductions (DPP): CTRL 0xB1 and 0x4E swap
// lanes 1 and 2 apart inside a quad, 0x141 mirrors each half-row of 8 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_lanes(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// kMagic + rint(x / sf) for a binary16 x (see above): one fma gives it except
// at an exact tie, where the exact remainder is +-sf/2 and k moves to the
// even neighbour. Used per group (zero-point), not per weight.
__device__ __forceinline__ float rint_quotient(float x, float sf, float inv, float half)
{
    constexpr float kMagic = 12582912.0f;
    const float k = fmaf(x, inv, kMagic) - kMagic;
    const float r = fmaf(-k, sf, x);
    const bool odd = (((int)k) & 1) != 0;   // -lo / sf <= 23 for the zero-point
    return (fabsf(r) == half && odd) ? k + (r > 0.0f ? 1.0f : -1.0f) : k;
}

template <int LPG, bool SYM>
__global__ __launch_bounds__(kThreads) void q4_quantize_pack_kernel(
    const uint16_t *__restrict__ W, int64_t K, int G, int blocks_per_row,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros)
{
    static_assert(LPG == 2 || LPG == 4 || LPG == 8, "lanes per group");
    constexpr int V = 16;                   // weights per lane
    constexpr int g = LPG * V;
    constexpr int GPB = kThreads / LPG;     // groups per block
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23: integers in its binade, low bits = value

    const int64_t n = blockIdx.x / blocks_per_row;
    const int c = blockIdx.x % blocks_per_row;
    const int t = threadIdx.x;
    const int gi = t / LPG, li = t % LPG;
    const int j = c * GPB + gi;
    const bool valid = j < G;
    const int64_t elem = n * K + (int64_t)j * g + li * V;

    u32x4 raw[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        raw[q] = u32x4{0u, 0u, 0u, 0u};
        if (valid) raw[q] = *reinterpret_cast<const u32x4 *>(W + elem + 8 * q);
    }
    // (each dword goes through a scalar first: __builtin_bit_cast of a vector
    // element reads element 0 with this compiler)
    half2v d[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; i++) {
        const uint32_t e = raw[i >> 2][i & 3];
        d[i] = __builtin_bit_cast(half2v, e);
    }

    // group statistics: (lo, -hi) as one fp16 pair, min-reduced over the
    // group's lanes. Both paths let a NaN or an infinity through to the pair,
    // which flags the group: the symmetric one takes max |x| on the 16-bit
    // patterns (they order as the magnitudes, with the infinities and NaN
    // above every finite value), the asymmetric one the IEEE 754-2019
    // minimum / maximum (v_pk_minimum3_f16 / v_pk_maximum3_f16, which
    // propagate NaN, unlike min / max), and so do the lane reductions.
    half2v st;
    if (SYM) {
        u16x2 ab = __builtin_bit_cast(u16x2, __builtin_bit_cast(uint32_t, d[0]) & 0x7fff7fffu);
#pragma unroll
        for (int i = 1; i < V / 2; i++)
            ab = __builtin_elementwise_max(ab, __builtin_bit_cast(u16x2, __builtin_bit_cast(uint32_t, d[i]) & 0x7fff7fffu));
        const uint16_t m = ab[0] > ab[1] ? ab[0] : ab[1];
        st = half2v{(_Float16)0.0f, -__builtin_bit_cast(_Float16, m)};
    } else {
        half2v mn = d[0], mx = d[0];
#pragma unroll
        for (int i = 1; i < V / 2; i++) {
            mn = __builtin_elementwise_minimum(mn, d[i]);
            mx = __builtin_elementwise_maximum(mx, d[i]);
        }
        st = half2v{__builtin_elementwise_minimum(mn[0], mn[1]), -__builtin_elementwise_maximum(mx[0], mx[1])};
    }
    st = __builtin_elementwise_minimum(st, __builtin_bit_cast(half2v, dpp_lanes<0xB1>(__builtin_bit_cast(uint32_t, st))));
    if (LPG >= 4)
        st = __builtin_elementwise_minimum(st, __builtin_bit_cast(half2v, dpp_lanes<0x4E>(__builtin_bit_cast(uint32_t, st))));
    if (LPG >= 8)
        st = __builtin_elementwise_minimum(st, __builtin_bit_cast(half2v, dpp_lanes<0x141>(__builtin_bit_cast(uint32_t, st))));
    // a group holding a NaN or an infinity is flagged: its scale is the fp16
    // NaN and its codes and zero-point are 0 (the arithmetic below then runs
    // on an all-zero group)
    const bool bad = !((float)st[0] >= -65504.0f && -(float)st[1] <= 65504.0f);
    const float lo = bad ? 0.0f : fminf((float)st[0], 0.0f);
    const float hi = bad ? 0.0f : fmaxf(-(float)st[1], 0.0f);   // SYM: max |x|

    const float s32 = SYM ? hi / 7.0f : (hi - lo) / 15.0f;   // IEEE division: rounded to fp16 next
    uint16_t s16 = f2h(s32);
    if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;   // 1.0
    const float sf = h2f(s16);
    const float inv = __builtin_amdgcn_rcpf(sf);
    const float half = 0.5f * sf;
    float zp = 8.0f;
    if (!SYM) zp = fminf(fmaxf(rint_quotient(-lo, sf, inv, half), 0.0f), 15.0f);
    const float mz = kMagic + zp;

    // codes: kMagic + zp + rint(x / sf), ties fixed per run of 8, clamped to [0, 15]
    float tq[V];
#pragma unroll
    for (int h8 = 0; h8 < V / 8; h8++) {
        bool tie = false;
#pragma unroll
        for (int i = 8 * h8; i < 8 * h8 + 8; i++) {
            const float x = (float)d[i >> 1][i & 1];
            tq[i] = fmaf(x, inv, mz);
            const float r = fmaf(-(tq[i] - mz), sf, x);
            tie |= fabsf(r) == half;
        }
        if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
            for (int i = 8 * h8; i < 8 * h8 + 8; i++) {
                const float x = (float)d[i >> 1][i & 1];
                const float k = tq[i] - mz;
                const float r = fmaf(-k, sf, x);
                const bool odd = fabsf(k) < 16777216.0f && (((int)k) & 1) != 0;
                if (fabsf(r) == half && odd) tq[i] += r > 0.0f ? 1.0f : -1.0f;
            }
        }
    }
    uint32_t b[V / 2];
#pragma unroll
    for (int p = 0; p < V / 2; p++) {
        const uint32_t e = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(tq[2 * p], kMagic, kMagic + 15.0f));
        const uint32_t o = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(tq[2 * p + 1], kMagic, kMagic + 15.0f));
        b[p] = (o << 4) | e;   // low byte: code 2p | code 2p+1 << 4 (the magic's low 12 bits are 0)
    }
    u32x2 word;
#pragma unroll
    for (int w = 0; w < 2; w++) {
        const uint32_t lo2 = __builtin_amdgcn_perm(b[4 * w + 1], b[4 * w], 0x0c0c0400u);
        const uint32_t hi2 = __builtin_amdgcn_perm(b[4 * w + 3], b[4 * w + 2], 0x0c0c0400u);
        word[w] = __builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
    }
    if (bad) {
        word = u32x2{0u, 0u};
        s16 = 0x7e00u;
    }
    if (valid) {
        *reinterpret_cast<u32x2 *>(codes + elem / 2) = word;
        if (li == 0) scales[n * G + j] = s16;
    }
    if (!SYM) {
        // zero-points of groups 2i and 2i + 1 meet through a lane swizzle
        // (xor LPG: the partner group's lanes); a missing last group packs 0
        const int z = valid && !bad ? (int)zp : 0;
        const int zo = __builtin_amdgcn_ds_swizzle(z, (LPG << 10) | 0x1F);
        if (li == 0 && (gi & 1) == 0 && valid)
            zeros[n * ((G + 1) / 2) + (j >> 1)] = (uint8_t)(z | (zo << 4));
    }
}

template <int LPG>
hipError_t launch_q4_g(const uint16_t *W, int64_t N, int64_t K, int sym, uint8_t *codes,
                       uint16_t *scales, uint8_t *zeros, hipStream_t st)
{
    constexpr int GPB = kThreads / LPG;
    const int G = (int)(K / (LPG * 16));
    const int per_row = (G + GPB - 1) / GPB;
    const int64_t blocks = N * per_row;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (sym)
        q4_quantize_pack_kernel<LPG, true><<<(unsigned)blocks, kThreads, 0, st>>>(
            W, K, G, per_row, codes, scales, zeros);
    else
        q4_quantize_pack_kernel<LPG, false><<<(unsigned)blocks, kThreads, 0, st>>>(
            W, K, G, per_row, codes, scales, zeros);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row INT8 (Operators guide §2.2 per-channel; the same arithmetic serves
// per-token activations): row values v = x * s (weights, DIV = false) or
// v = x / s (activations, DIV = true), scale = max(max|v|, 1e-8) / 127,
// q = clip(rne(v / scale), -127, 127). The generic kernel (rows wider than
// 8192) has one block per row, IEEE divisions, and reads the row twice; each
// lane owns 8-element chunks (16-byte loads, 8-byte stores).
// the block's maximum of |v| bit patterns (256 threads)
__device__ __forceinline__ uint32_t block_max_bits(uint32_t v, uint32_t *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return max(max(red[0], red[1]), max(red[2], red[3]));
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

template <bool FP8>
__device__ __forceinline__ u32x2 row_codes8(const float v[8], float scale)
{
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) q[i] = v[i] / scale;
    return u32x2{row_codes4<FP8>(q[0], q[1], q[2], q[3]), row_codes4<FP8>(q[4], q[5], q[6], q[7])};
}

template <bool FP8, bool DIV, int CPT>
__global__ __launch_bounds__(kThreads) void q8_rows_generic_kernel(const uint16_t *__restrict__ X,
                                                          const float *__restrict__ s,
                                                          int64_t K, uint8_t *__restrict__ Q,
                                                          float *__restrict__ scale_out)
{
    __shared__ uint32_t red[4];
    const int64_t r = blockIdx.x;
    const uint16_t *row = X + r * K;
    uint8_t *qrow = Q + r * K;
    const int64_t step = (int64_t)kThreads * 8;
    uint32_t ab = 0u;
    // a row holding a NaN or an infinity is flagged: NaN scale, codes 0
    if (CPT > 0) {
        float v[CPT > 0 ? CPT : 1][8];
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int64_t k0 = threadIdx.x * 8 + c * step;
            if (k0 < K) {
                load_row_chunk<DIV>(row, s, k0, v[c]);
#pragma unroll
                for (int i = 0; i < 8; i++) ab = max(ab, abs_bits(v[c][i]));
            }
        }
        ab = block_max_bits(ab, red);
        const bool bad = ab >= kNonFinite;
        const float scale = (bad ? 1.0f : fmaxf(__builtin_bit_cast(float, ab), 1e-8f)) / kRowMax<FP8>;
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int64_t k0 = threadIdx.x * 8 + c * step;
            if (k0 < K)
                *reinterpret_cast<u32x2 *>(qrow + k0) = bad ? u32x2{0u, 0u} : row_codes8<FP8>(v[c], scale);
        }
        if (threadIdx.x == 0) scale_out[r] = bad ? __builtin_nanf("") : scale;
    } else {
        float v[8];
        for (int64_t k0 = threadIdx.x * 8; k0 < K; k0 += step) {
            load_row_chunk<DIV>(row, s, k0, v);
#pragma unroll
            for (int i = 0; i < 8; i++) ab = max(ab, abs_bits(v[i]));
        }
        ab = block_max_bits(ab, red);
        const bool bad = ab >= kNonFinite;
        const float scale = (bad ? 1.0f : fmaxf(__builtin_bit_cast(float, ab), 1e-8f)) / kRowMax<FP8>;
        for (int64_t k0 = threadIdx.x * 8; k0 < K; k0 += step) {
            load_row_chunk<DIV>(row, s, k0, v);
            *reinterpret_cast<u32x2 *>(qrow + k0) = bad ? u32x2{0u, 0u} : row_codes8<FP8>(v, scale);
        }
        if (threadIdx.x == 0) scale_out[r] = bad ? __builtin_nanf("") : scale;
    }
}

// max over each half-wavefront (lanes 0-31 and 32-63 each end with their own):
// DPP quad swaps, half-row and row mirrors, then a lane swizzle across 16
// (a holds |v| bits: they order as the magnitudes with NaN and the
// infinities on top, so the lanes meet with integer max)
__device__ __forceinline__ float halfwave_max(float a)
{
    auto dpp = [](uint32_t v, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctrl)::value, 0xF, 0xF, false);
    };
    uint32_t b = __builtin_bit_cast(uint32_t, a);
    b = max(b, dpp(b, std::integral_constant<int, 0xB1>{}));
    b = max(b, dpp(b, std::integral_constant<int, 0x4E>{}));
    b = max(b, dpp(b, std::integral_constant<int, 0x141>{}));
    b = max(b, dpp(b, std::integral_constant<int, 0x140>{}));
    b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (16 << 10) | 0x1F));
    return __builtin_bit_cast(float, b);
}

// Per-row INT8 for rows of at most 8192 values: a block of T threads owns
// RPB rows and each thread the same CPT chunks of 8 columns in every row, so
// the per-column factor (the fp64 reciprocal of s for activations, s itself
// for weights) is formed once per block. Every load is issued up front and
// none is conditional (rows past M and chunks past K read clamped, valid
// addresses and are masked afterwards), so the compiler's waits stay partial
// and row rr is worked on as soon as its own bytes have landed. Per row: the
// values v, the block's max |v| (one LDS slot per row, one barrier), the
// scale by an IEEE fp32 division, and the codes rint(fl32(v / scale)) from
// one fp64 multiply.
template <bool FP8, bool DIV, bool HAS_S, int CPT, int RPB, int T>
__global__ __launch_bounds__(T) void q8_rows_kernel(const uint16_t *__restrict__ X,
                                                    const float *__restrict__ s, int64_t M,
                                                    int64_t K, uint8_t *__restrict__ Q,
                                                    float *__restrict__ scale_out)
{
    constexpr int HW = T / 32;   // half-wavefronts per block
    __shared__ float red[RPB][HW];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * RPB;
    constexpr int64_t step = (int64_t)T * 8;

    int64_t kc[CPT];
    bool kin[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c++) {
        const int64_t k0 = t * 8 + c * step;
        kin[c] = k0 < K;
        kc[c] = kin[c] ? k0 : K - 8;
    }
    // the column factors first (they are needed first), then the rows in order
    floatx4 slo[CPT], shi[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c++) {
        slo[c] = floatx4{1.f, 1.f, 1.f, 1.f};
        shi[c] = floatx4{1.f, 1.f, 1.f, 1.f};
        if (HAS_S) {
            slo[c] = *reinterpret_cast<const floatx4 *>(s + kc[c]);
            shi[c] = *reinterpret_cast<const floatx4 *>(s + kc[c] + 4);
        }
    }
    u32x4 raw[RPB][CPT];
#pragma unroll
    for (int rr = 0; rr < RPB; rr++) {
        const int64_t r = r0 + rr < M ? r0 + rr : M - 1;
#pragma unroll
        for (int c = 0; c < CPT; c++) raw[rr][c] = *reinterpret_cast<const u32x4 *>(X + r * K + kc[c]);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the arithmetic
    float sv[CPT][8];
    double rd[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; c++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            sv[c][i] = slo[c][i];
            sv[c][4 + i] = shi[c][i];
        }
        if (DIV && HAS_S) {
#pragma unroll
            for (int i = 0; i < 8; i++) rd[c][i] = recip64((double)sv[c][i]);
        }
    }

#pragma unroll
    for (int rr = 0; rr < RPB; rr++) {
        float v[CPT][8];
        uint32_t ab = 0u;
#pragma unroll
        for (int c = 0; c < CPT; c++) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t d = raw[rr][c][i >> 1];
                const float x = h2f((uint16_t)((i & 1) ? (d >> 16) : (d & 0xffffu)));
                if (!HAS_S) v[c][i] = x;
                else if (DIV) v[c][i] = (float)((double)x * rd[c][i]);   // fl32(x / s)
                else v[c][i] = x * sv[c][i];
            }
            uint32_t m = max(max(abs_bits(v[c][0]), abs_bits(v[c][1])), abs_bits(v[c][2]));
            m = max(max(m, abs_bits(v[c][3])), abs_bits(v[c][4]));
            m = max(max(m, abs_bits(v[c][5])), abs_bits(v[c][6]));
            m = max(m, abs_bits(v[c][7]));
            if (kin[c]) ab = max(ab, m);   // chunks past K hold a clamped copy: not counted
        }
        float a = halfwave_max(__builtin_bit_cast(float, ab));
        if ((lane & 31) == 0) red[rr][wave * 2 + (lane >> 5)] = a;
        __syncthreads();
#pragma unroll
        for (int h = 0; h < HW; h += 4) {
            const u32x4 m = *reinterpret_cast<const u32x4 *>(&red[rr][h]);   // maxima as bits
            const uint32_t m0 = m[0], m1 = m[1], m2 = m[2], m3 = m[3];
            a = __builtin_bit_cast(float, max(__builtin_bit_cast(uint32_t, a), max(max(m0, m1), max(m2, m3))));
        }
        // a row holding a NaN or an infinity is flagged: NaN scale, codes 0
        const bool bad = __builtin_bit_cast(uint32_t, a) >= kNonFinite;
        a = bad ? 1.0f : fmaxf(a, 1e-8f);
        const float scale = a / kRowMax<FP8>;
        const double rs = recip64((double)scale);
        const int64_t r = r0 + rr;
        if (r < M) {
#pragma unroll
            for (int c = 0; c < CPT; c++) {
                float q[8];
#pragma unroll
                for (int i = 0; i < 8; i++) q[i] = (float)((double)v[c][i] * rs);   // fl32(v / scale)
                u32x2 out = {row_codes4<FP8>(q[0], q[1], q[2], q[3]), row_codes4<FP8>(q[4], q[5], q[6], q[7])};
                if (bad) out = u32x2{0u, 0u};
                if (kin[c]) *reinterpret_cast<u32x2 *>(Q + r * K + kc[c]) = out;
            }
            if (t == 0) scale_out[r] = bad ? __builtin_nanf("") : scale;
        }
    }
}

template <bool FP8, bool DIV>
hipError_t launch_q8_rows(const uint16_t *X, const float *s, int64_t rows, int64_t K, uint8_t *Q,
                          float *scale, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int RPB = 4, T = 512;
    const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
    if (K <= 4096) {
        if (s) q8_rows_kernel<FP8, DIV, true, 1, RPB, T><<<grid, T, 0, st>>>(X, s, rows, K, Q, scale);
        else q8_rows_kernel<FP8, DIV, false, 1, RPB, T><<<grid, T, 0, st>>>(X, s, rows, K, Q, scale);
    } else if (K <= 8192) {
        if (s) q8_rows_kernel<FP8, DIV, true, 2, RPB, T><<<grid, T, 0, st>>>(X, s, rows, K, Q, scale);
        else q8_rows_kernel<FP8, DIV, false, 2, RPB, T><<<grid, T, 0, st>>>(X, s, rows, K, Q, scale);
    } else   // wider rows: one row per block, the row read twice
        q8_rows_generic_kernel<FP8, DIV, 0><<<(unsigned)rows, kThreads, 0, st>>>(X, s, K, Q, scale);
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
    case 32: return launch_q4_g<2>(W, N, K, sym, codes, scales, zeros, st);
    case 64: return launch_q4_g<4>(W, N, K, sym, codes, scales, zeros, st);
    case 128: return launch_q4_g<8>(W, N, K, sym, codes, scales, zeros, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_q8_weight(const uint16_t *W, const float *s, int64_t N, int64_t K, int8_t *Wq,
                            float *sw, hipStream_t st)
{
    return launch_q8_rows<false, false>(W, s, N, K, reinterpret_cast<uint8_t *>(Wq), sw, st);
}

hipError_t launch_q8_act(const uint16_t *X, const float *s, int64_t M, int64_t K, int8_t *Xq,
                         float *sx, hipStream_t st)
{
    return launch_q8_rows<false, true>(X, s, M, K, reinterpret_cast<uint8_t *>(Xq), sx, st);
}

hipError_t launch_fp8_weight(const uint16_t *W, const float *s, int64_t N, int64_t K, uint8_t *Wq,
                             float *sw, hipStream_t st)
{
    return launch_q8_rows<true, false>(W, s, N, K, Wq, sw, st);
}

hipError_t launch_fp8_act(const uint16_t *X, const float *s, int64_t M, int64_t K, uint8_t *Xq,
                          float *sx, hipStream_t st)
{
    return launch_q8_rows<true, true>(X, s, M, K, Xq, sx, st);
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
