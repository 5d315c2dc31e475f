// W4A16 linear layer on gfx950: Y[M,N] = X[M,K] * W_hat[N,K]^T with the INT4
// weight dequantized inside the GEMM (Quantization operators guide,
// blog.freezetheflame.cc, §1.2: quantize / compute / dequantize fused into
// the GEMM; Core ideas, ai-infra.cypggs.com, §2.2: w_hat = (u - zp) * s;
// Method boundaries, llm-glossary.tokens-kit.com, GPTQ section: decode is
// bound by the weight read, prefill by the dequant + matrix-core path).
// This file holds the dispatch and the kernels for M > 16; the decode GEMV
// (M <= 16, g = 128) is in w4a16_gemv.hip.
//
// Arithmetic. The skinny and 128 x 128 kernels feed v_mfma_f32_16x16x32_f16
// with the exact integers (u - zp) in fp16 (unpacked as in w4a16_dequant.hpp)
// and x in fp16: every product is exact in fp32. The fp32 partial sum of one
// 128-wide k-block is multiplied by the fp32 value of the block's group scale
// and added to the fp32 total. The large-M kernel dequantizes to fp16
// (u - zp) * s once per weight (one rounding) and accumulates in fp32.
//
// The packed weight is read in place in the layout q4_quantize_pack writes
// (row-major codes [N, K/2], scales [N, K/g], zeros [N, ceil(K/g/2)]); it is
// never expanded in memory.
#include <cstdlib>

#include "fp4_codes.hpp"
#include "nf4_lut.hpp"
#include "w4a16_dequant.hpp"

namespace q4k {
namespace {

// Tuning override for the large-M GEMM: Q4_GEMM_NU=4|8|11 forces the tile
// width (32 NU columns). Read at every call.
int gemm_nu_override()
{
    const char *e = std::getenv("Q4_GEMM_NU");
    const int v = e ? std::atoi(e) : 0;
    return (v == 4 || v == 8 || v == 11) ? v : 0;
}

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Skinny kernel, M <= 64 (decode and batched decode). Memory bound: the
// packed weight is streamed once with 16-byte loads, dequantized in registers
// and fed to the MFMA with X as the A operand (rows m) and the weight as the
// B operand (columns n). A block owns NT*16 output channels and all of K; its
// 4 wavefronts split the k-blocks, issue PF k-blocks of code loads at a time,
// and meet in LDS for the final sum. X fragments come from L2.
template <int MT, int NT, int PF>
__global__ __launch_bounds__(kThreads) void w4a16_skinny_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, int g, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    __shared__ float red[4][MT * NT * 4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int KB = K >> 7;
    const int kb_begin = (KB * wave) >> 2, kb_end = (KB * (wave + 1)) >> 2;
    const int n_base = blockIdx.x * (NT * 16);
    const int G = K / g, Gz = (G + 1) >> 1, bpg = g >> 7;
    const int64_t row_bytes = K >> 1;

    int64_t nrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const int n = n_base + nt * 16 + r16;
        nrow[nt] = n < N ? n : N - 1;
    }
    const uint16_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int m = mt * 16 + r16;
        xok[mt] = m < M;
        xrow[mt] = X + (int64_t)(xok[mt] ? m : 0) * K + q * 32;
    }

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += PF) {
        u32x4 cw[PF][NT];
        float sc[PF][NT];
        ZeroConst zb[PF][NT];
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int kb = kb0 + p;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                if (kb < kb_end) {
                    const int grp = kb / bpg;
                    cw[p][nt] = *reinterpret_cast<const u32x4 *>(codes + nrow[nt] * row_bytes +
                                                                 kb * 64 + q * 16);
                    sc[p][nt] = scale16(scales[nrow[nt] * G + grp]);
                    zb[p][nt] = zero_const(group_zp(zeros, nrow[nt], Gz, grp));
                } else {
                    cw[p][nt] = u32x4{0u, 0u, 0u, 0u};
                    sc[p][nt] = 0.0f;
                    zb[p][nt] = zero_const(0);
                }
            }
        }
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int kb = kb0 + p;
            if (kb >= kb_end) break;
            floatx4 part[MT][NT];
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++) part[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                half8 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    u32x4 d = {0u, 0u, 0u, 0u};
                    if (xok[mt]) d = *reinterpret_cast<const u32x4 *>(xrow[mt] + kb * 128 + t * 8);
                    a[mt] = __builtin_bit_cast(half8, permute_x(d));
                }
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    const half8 b = dequant8(cw[p][nt][t], zb[p][nt]);
#pragma unroll
                    for (int mt = 0; mt < MT; mt++)
                        part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], b, part[mt][nt],
                                                                              0, 0, 0);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[mt][nt][r] = fmaf(part[mt][nt][r], sc[p][nt], acc[mt][nt][r]);
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int r = 0; r < 4; r++) red[wave][(mt * NT + nt) * 4 + r][lane] = acc[mt][nt][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * NT * 4 * 64; idx += kThreads) {
        const int reg = idx >> 6, l = idx & 63;
        const float v = red[0][reg][l] + red[1][reg][l] + red[2][reg][l] + red[3][reg][l];
        const int mt = reg / (NT * 4), nt = (reg >> 2) % NT, r = reg & 3;
        const int m = mt * 16 + 4 * (l >> 4) + r;
        const int n = n_base + nt * 16 + (l & 15);
        if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(v);
    }
}

// ---------------------------------------------------------------------------
// Small-group kernel: any g that is a multiple of 32 (the quantizer writes
// g = 32 and 64; Core ideas, ai-infra.cypggs.com, §2.3 granularity table),
// K a multiple of g, any M. Work advances in 32-wide k steps; a step never
// straddles two groups, so its MFMA sums one group only and the group's
// scale multiplies the step's exact fp32 partial sum, as in the kernels
// above. Lane (r16, q) takes k = 32 s + 8 q .. + 7 of step s for both
// operands: one code dword (eight nibbles) and 16 bytes of X. A block owns
// NT * 16 output channels and 16 MT rows of Y (grid.y walks the rows); its
// 4 wavefronts split the steps and meet in LDS for the final sum.
template <int MT, int NT, int PF>
__global__ __launch_bounds__(kThreads) void w4a16_subg_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, int g, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    __shared__ float red[4][MT * NT * 4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int S = K >> 5;                                       // 32-wide steps
    const int s_begin = (S * wave) >> 2, s_end = (S * (wave + 1)) >> 2;
    const int n_base = blockIdx.x * (NT * 16), m_base = blockIdx.y * (MT * 16);
    const int G = K / g, Gz = (G + 1) >> 1, spg = g >> 5;      // steps per group
    const int64_t row_bytes = K >> 1;

    int64_t nrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const int n = n_base + nt * 16 + r16;
        nrow[nt] = n < N ? n : N - 1;
    }
    const uint16_t *xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int m = m_base + mt * 16 + r16;
        xrow[mt] = X + (int64_t)(m < M ? m : M - 1) * K + q * 8;   // rows past M repeat M - 1
    }

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = s_begin; s0 < s_end; s0 += PF) {
        uint32_t cw[PF][NT];
        float sc[PF][NT];
        ZeroConst zb[PF][NT];
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int s = s0 + p < s_end ? s0 + p : s_end - 1;   // past the end: reloaded, unused
            const int grp = s / spg;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                cw[p][nt] = *reinterpret_cast<const uint32_t *>(codes + nrow[nt] * row_bytes + s * 16 + q * 4);
                sc[p][nt] = scale16(scales[nrow[nt] * G + grp]);
                zb[p][nt] = zero_const(group_zp(zeros, nrow[nt], Gz, grp));
            }
        }
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int s = s0 + p;
            if (s >= s_end) break;
            half8 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
                a[mt] = __builtin_bit_cast(half8, permute_x(*reinterpret_cast<const u32x4 *>(xrow[mt] + s * 32)));
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const half8 b = dequant8(cw[p][nt], zb[p][nt]);
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    const floatx4 part = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a[mt], b, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[mt][nt][r] = fmaf(part[r], sc[p][nt], acc[mt][nt][r]);
                }
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int r = 0; r < 4; r++) red[wave][(mt * NT + nt) * 4 + r][lane] = acc[mt][nt][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * NT * 4 * 64; idx += kThreads) {
        const int reg = idx >> 6, l = idx & 63;
        const float v = red[0][reg][l] + red[1][reg][l] + red[2][reg][l] + red[3][reg][l];
        const int mt = reg / (NT * 4), nt = (reg >> 2) % NT, r = reg & 3;
        const int m = m_base + mt * 16 + 4 * (l >> 4) + r;
        const int n = n_base + nt * 16 + (l & 15);
        if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(v);
    }
}

// ---------------------------------------------------------------------------
// Prefill kernel, M > 64. Compute bound. A 256-thread block computes a
// 128 x 128 tile of Y; its 4 wavefronts form a 2 x 2 grid of 64 x 64
// sub-tiles (4 x 4 MFMA tiles each). Per 128-wide k-block: the X tile and the
// packed weight tile are loaded from HBM into registers one k-block ahead,
// stored to LDS (X permuted to the operand k order, the weight dequantized
// to exact fp16 (u - zp) once per block, not once per wavefront), and the
// group scale of each weight row goes to LDS beside them.
constexpr int PBM = 128, PBN = 128, PLD = 128 + 8;   // LDS row stride in halves

__global__ __launch_bounds__(kThreads, 2) void w4a16_prefill_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, int g, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) _Float16 Xs[PBM][PLD];
    __shared__ __attribute__((aligned(16))) _Float16 Ws[PBN][PLD];
    __shared__ float Ss[PBN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.y * PBM, n0 = blockIdx.x * PBN;
    const int KB = K >> 7, G = K / g, Gz = (G + 1) >> 1, bpg = g >> 7;
    const int64_t row_bytes = K >> 1;

    // global -> register assignment
    const int xc = tid & 15, xr0 = tid >> 4;     // X: 16 chunks of 8 halves per row, 8 rows/thread
    const int cc = tid & 3, cr0 = tid >> 2;      // codes: 4 chunks of 16 bytes per row, 2 rows/thread
    u32x4 xreg[8], creg[2];
    ZeroConst zreg[2];
    float sreg = 0.0f;

    auto load_tile = [&](int kb) {
        const int grp = kb / bpg;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int m = m0 + xr0 + 16 * i;
            xreg[i] = u32x4{0u, 0u, 0u, 0u};
            if (m < M)
                xreg[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * K + kb * 128 + xc * 8);
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            int n = n0 + cr0 + 64 * i;
            n = n < N ? n : N - 1;
            creg[i] = *reinterpret_cast<const u32x4 *>(codes + (int64_t)n * row_bytes + kb * 64 +
                                                       cc * 16);
            zreg[i] = zero_const(group_zp(zeros, n, Gz, grp));
        }
        if (tid < PBN) {
            int n = n0 + tid;
            n = n < N ? n : N - 1;
            sreg = scale16(scales[(int64_t)n * G + grp]);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 8; i++)
            *reinterpret_cast<u32x4 *>(&Xs[xr0 + 16 * i][xc * 8]) = permute_x(xreg[i]);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int t4 = 0; t4 < 4; t4++)
                *reinterpret_cast<half8 *>(&Ws[cr0 + 64 * i][cc * 32 + t4 * 8]) =
                    dequant8(creg[i][t4], zreg[i]);
        if (tid < PBN) Ss[tid] = sreg;
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 4; nt++) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    load_tile(0);
    for (int kb = 0; kb < KB; ++kb) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kb + 1 < KB) load_tile(kb + 1);
        floatx4 part[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int nt = 0; nt < 4; nt++) part[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            half8 a[4], b[4];
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
                a[mt] = *reinterpret_cast<const half8 *>(&Xs[wm * 64 + mt * 16 + r16][q * 32 + t * 8]);
#pragma unroll
            for (int nt = 0; nt < 4; nt++)
                b[nt] = *reinterpret_cast<const half8 *>(&Ws[wn * 64 + nt * 16 + r16][q * 32 + t * 8]);
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
#pragma unroll
                for (int nt = 0; nt < 4; nt++)
                    part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], b[nt], part[mt][nt],
                                                                          0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const float s = Ss[wn * 64 + nt * 16 + r16];
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[mt][nt][r] = fmaf(part[mt][nt][r], s, acc[mt][nt][r]);
        }
    }

#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 4; nt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = m0 + wm * 64 + mt * 16 + 4 * q + r;
                const int n = n0 + wn * 64 + nt * 16 + r16;
                if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(acc[mt][nt][r]);
            }
}

// ---------------------------------------------------------------------------
// Batched decode, 1 < M <= 64, g = 128. A block of 4 wavefronts owns 64
// output channels; wavefront w owns 16 of them (one MFMA column tile) across
// all of K, so no wavefront waits on another's partial sums. X is the operand
// all four share: one k-block of it (16 MT rows x 128 k, rows past M repeat
// row M - 1) at a time goes straight from global memory into an R-slot LDS
// ring with direct-to-LDS loads issued R - 1 k-blocks ahead; its 16-byte
// chunks are XOR-swizzled (chunk c of row m at c ^ xswz(m)) so the
// fragment reads, 16 rows of one chunk, are conflict-free. Each wavefront
// streams its own code runs, scales and zero-points through a DC-deep
// register ring. One barrier per k-block: before it every wavefront waits
// for its share of the k-block's X (the wait counts are fixed: past the end
// the last k-block is fetched again into slots nobody reads).
// Natural k order: lane (r16, q) takes k = 32 q .. 32 q + 31 of each k-block
// for both operands; MFMA step t pairs dword t of its code run with
// X[m][32 q + 8 t .. + 7]. Unpack (exact, natural order, 3 operations per
// pair): v_perm copies byte p of a code dword into bytes 0 and 2, one
// v_and_or lifts its low nibble to bit 0 of the low fp16 half (1024 + u0) and
// its high nibble to bit 4 of the high half (1024 + 16 u1), and one packed fma
// with (1, 1/16) and (-(1024 + zp), -(64 + zp)) leaves (u0 - zp, u1 - zp).
// Each product x (u - zp) is exact in fp32; the fp32 partial sum of a k-block
// is scaled by its group scale in fp32.
// Swizzle of the X tiles of the batched kernels: the 16-byte chunk c of a
// 256-byte row r is stored at c ^ xswz(r). A 16-lane fragment read touches
// one chunk of 16 rows. On gfx950 a ds_read_b128 serves 16 lanes per cycle,
// four groups of four lanes that share lane bit 5 and the parity of lane
// bits 2-4 (lanes 0-3, 12-15, 20-23, 24-27 together), and 16 bytes of a
// 256-byte bank row per lane (the grouping was fitted to the bank-conflict
// counter on a set of probe patterns). With c ^ r the four lanes of a group
// with row bits 2 and 3 swapped for q land on the same chunk (two-way
// conflicts on every read); c ^ (r & 11) keeps every group on 16 distinct
// chunks for each of the four MFMA steps.
__device__ __forceinline__ int xswz(int r) { return r & 11; }

__device__ __forceinline__ uint32_t unpack_pair(uint32_t w, int p, uint32_t zadd)
{
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x01010101u * (uint32_t)p);
    const half2v x = __builtin_bit_cast(half2v, and_or(t, 0x00F0000Fu, 0x64006400u));
    const half2v mul = __builtin_bit_cast(half2v, 0x2C003C00u);   // (1, 1/16)
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(x, mul, __builtin_bit_cast(half2v, zadd)));
}

template <int MT, int KS, int R, int DC, bool ASYM>
__global__ __launch_bounds__(256 * KS) void w4a16_batched_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    static_assert(MT <= 4 && R <= 4 && DC <= 16 && KS * R * MT <= 32, "ring sizes");
    constexpr int SLOT = MT * 16 * 256;          // bytes of one k-block of X
    constexpr int LPC = ASYM ? 3 : 2;            // loads per code-ring refill
    // (fixed-size arrays: arrays sized by a template parameter and captured by
    // the lambdas below make this compiler drop the kernel's host stub)
    __shared__ __attribute__((aligned(1024))) unsigned char xs[32 * 16 * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave & 3, ks = wave >> 2;     // column tile, k-split group
    const int r16 = lane & 15, q = lane >> 4;
    const int KBS = (K >> 7) / KS;               // k-blocks per group
    const int kbase = ks * KBS;
    // every block walks its k-blocks from a different start, so that at any
    // moment the blocks read different parts of X (all starting at the same
    // k-block would put every block on the same few L2 lines at once)
    const int rot = (int)(blockIdx.x % (unsigned)KBS);
    auto kblock = [&](int kb) {   // iteration -> global k-block (kb may be past the end)
        const int kk = (kb < KBS ? kb : KBS - 1) + rot;
        return kbase + (kk < KBS ? kk : kk - KBS);
    };
    const uint32_t G = (uint32_t)(K >> 7), Gz = (G + 1) >> 1, kh = (uint32_t)K >> 1;
    const int n = blockIdx.x * 64 + wn * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    unsigned char *ring = xs + ks * R * SLOT;

    // direct-to-LDS X loads: instruction j of wavefront wn fills rows
    // 4 (4 j + wn) .. + 3 of a slot; lane i: row 4 (4 j + wn) + i / 16, stored
    // chunk i % 16, logical chunk (i % 16) ^ xswz(row % 16)
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < MT; j++) {
        const int m = 4 * (4 * j + wn) + (lane >> 4);
        const int c = (lane & 15) ^ xswz(m);
        xoff[j] = ((uint32_t)(m < M ? m : M - 1) * (uint32_t)K + 8u * (uint32_t)c) * 2u;
    }
    const unsigned char *Xb = reinterpret_cast<const unsigned char *>(X);
    auto issue_x = [&](int kb) {   // kb >= 0: the group's kb-th iteration
        const int kc = kblock(kb);
        unsigned char *slot = ring + (kb % R) * SLOT;
#pragma unroll
        for (int j = 0; j < MT; j++)
            __builtin_amdgcn_global_load_lds(Xb + xoff[j] + (uint32_t)kc * 256u, slot + (4 * j + wn) * 1024,
                                             16, 0, 0);
    };
    u32x4 cw[16];
    uint32_t sc[16], zb[16];
    auto issue_w = [&](int kb) {
        const int kc = kblock(kb);
        cw[kb % DC] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)kc * 64u + q * 16u));
        sc[kb % DC] = scales[nrow * G + kc];
        if (ASYM) zb[kb % DC] = zeros[nrow * Gz + (kc >> 1)];
    };
    auto wait_x = [&]() {   // this wavefront's share of the oldest X slot has landed
        asm volatile("" ::: "memory");
        Q4_WAIT_VM_LGKM0(LPC + (R - 2) * (MT + LPC));
    };

    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One issue step per k-block: X of k-block i + R - 1, then the code run,
    // scale and zero-point of k-block i + DC - 1, in that order (the fences
    // keep the compiler from reordering the two groups, which the fixed wait
    // counts rely on). The prologue runs the same steps for i = -(DC - 1) ..
    // -1 (X indices below 0 fetch k-block 0 into slot 0 again), so the loop
    // head sees one pattern of outstanding loads from both sides.
    auto step_issue = [&](int i) {
        asm volatile("" ::: "memory");
        issue_x(i + R - 1 < 0 ? 0 : i + R - 1);
        asm volatile("" ::: "memory");
        issue_w(i + DC - 1);
        asm volatile("" ::: "memory");
    };
#pragma unroll
    for (int i = -(DC - 1); i < 0; i++) step_issue(i);
    // the group's k-blocks are a multiple of DC (and DC of R): ring slots are
    // compile-time; every group runs the same number of steps, so the block
    // barrier serves all of them
    for (int kb0 = 0; kb0 < KBS; kb0 += DC) {
#pragma unroll
        for (int u = 0; u < DC; u++) {
            const int kb = kb0 + u;
            wait_x();
            __builtin_amdgcn_s_barrier();
            step_issue(kb);
            const unsigned char *slot = ring + (kb % R) * SLOT;
            const int kg = kblock(kb);
            const uint32_t zp = ASYM ? (zb[u] >> (4 * (kg & 1))) & 15u : 8u;
            const uint32_t zadd = (0xE400u + zp) | ((0xD400u + 16u * zp) << 16);   // 1 at 1024, 1/16 at 64
            floatx4 part[MT];
#pragma unroll
            for (int mt = 0; mt < MT; mt++) part[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t w = cw[u][t];
                const u32x4 bv = {unpack_pair(w, 0, zadd), unpack_pair(w, 1, zadd),
                                  unpack_pair(w, 2, zadd), unpack_pair(w, 3, zadd)};
                const half8 b = __builtin_bit_cast(half8, bv);
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    const int m = mt * 16 + r16;
                    const half8 a = *reinterpret_cast<const half8 *>(slot + m * 256 + 16 * ((4 * q + t) ^ xswz(r16)));
                    part[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, part[mt], 0, 0, 0);
                }
            }
            const float s = h2f((uint16_t)sc[u]);
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[mt][r] = fmaf(part[mt][r], s, acc[mt][r]);
        }
    }
    Q4_WAIT_VM_LGKM0(0);   // the refetches past the end

    if (KS > 1) {
        // the k-split groups' partial sums meet in LDS (group order fixed)
        float *red = reinterpret_cast<float *>(xs);   // [KS - 1][4 wn][MT * 4][64]
        __syncthreads();
        if (ks > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) red[(((ks - 1) * 4 + wn) * MT * 4 + mt * 4 + r) * 64 + lane] = acc[mt][r];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; g2++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[mt][r] += red[(((g2 - 1) * 4 + wn) * MT * 4 + mt * 4 + r) * 64 + lane];
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = mt * 16 + 4 * q + r;
            if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(acc[mt][r]);
        }
}

// ---------------------------------------------------------------------------
// Batched decode, 16 < M <= 64, with the wavefront's whole weight slice in
// registers. The ring kernel above keeps only R - 1 k-blocks of code runs in
// flight per row, so HBM sees each 2 KB weight row as 64-byte pieces spread
// over the whole kernel, and a step costs about one memory latency over the
// ring depth. Here each of the 4 KS compute wavefronts issues the code runs,
// scales and zero-points of all its KBS (<= 16) k-blocks at once, so the
// weight streams at the rate of the decode GEMV, and X (L2-resident) goes
// through an R-slot LDS ring per k-split group that a wavefront of its own
// fills: memory loads complete in order, so a compute wavefront that also
// issued X loads would have to wait for all of its code runs before its
// first X slot, and every MFMA would follow the weight stream instead of
// overlapping it. With the loads split, step i waits only for the code run
// of its own k-block (the compiler's in-order count) and for the block
// barrier after which the loader has seen slot i land. Same operand order,
// unpack and arithmetic as the ring kernel.
template <int MT, int KS, int R, int KBS, bool ASYM, int NT, int GS = 128>
__global__ __launch_bounds__(64 * (NT + 1) * KS) void w4a16_batched_cres_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    constexpr int XI = MT * 4;                   // loader instructions per slot (1 KB each)
    constexpr int CD = 5;                        // k-blocks of code runs in flight per wavefront
    static_assert(GS == 32 || GS == 64 || GS == 128, "group sizes");
    constexpr int GPK = 128 / GS;                // groups per 128-wide k-block
    constexpr int NS = KBS * GPK;                // groups of the wavefront's k-blocks
    static_assert(MT <= 4 && KS * R * MT <= 32 && (KBS == 8 || KBS == 16) && (R - 2) * XI <= 63, "ring sizes");
    constexpr int SLOT = MT * 16 * 256;          // bytes of one k-block of X
    __shared__ __attribute__((aligned(1024))) unsigned char xs[32 * 16 * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool loader = wave >= NT * KS;         // waves NT KS .. (NT + 1) KS - 1 fill the X rings
    const int wn = wave % NT, ks = loader ? wave - NT * KS : wave / NT;   // column tile, k-split group
    const int r16 = lane & 15, q = lane >> 4;
    const int kbase = ks * KBS;
    auto kblock = [&](int i) { return kbase + (i < KBS ? i : KBS - 1); };   // i may be past the end
    const uint32_t G = (uint32_t)(K / GS), Gz = (G + 1) >> 1, kh = (uint32_t)K >> 1;
    unsigned char *ring = xs + ks * R * SLOT;

    if (loader) {
        // Slot j of the ring holds k-block kblock(j) of X, rows 0 .. 16 MT - 1
        // (rows past M repeat row M - 1), 16 chunks of 16 bytes per row.
        // Direct-to-LDS instruction e puts lane i at slot byte 1024 e + 16 i:
        // chunk c = 64 e + i is row c / 16, stored chunk c % 16, logical chunk
        // (c % 16) ^ xswz(row % 16).
        // (a fixed-size array: one sized by a template parameter and captured
        // by the lambda below makes this compiler drop the kernel's host stub)
        uint32_t xoff[16];
#pragma unroll
        for (int e = 0; e < XI; e++) {
            const int m = (64 * e + lane) >> 4;
            const int c = (lane & 15) ^ xswz(m & 15);
            xoff[e] = ((uint32_t)(m < M ? m : M - 1) * (uint32_t)K + 8u * (uint32_t)c) * 2u;
        }
        const unsigned char *Xb = reinterpret_cast<const unsigned char *>(X);
        auto issue_x = [&](int i) {
            const int kc = kblock(i);
            unsigned char *slot = ring + (i % R) * SLOT;
#pragma unroll
            for (int e = 0; e < XI; e++)
                __builtin_amdgcn_global_load_lds(Xb + xoff[e] + (uint32_t)kc * 256u, slot + e * 1024, 16, 0, 0);
        };
#pragma unroll
        for (int i = 0; i < R - 1; i++) issue_x(i);
        // the compute wavefronts issue their code runs after this barrier, so
        // the first X slots are ahead of the weight stream in the queues
        __builtin_amdgcn_s_barrier();
        // step i: slot i has landed once at most the later slots issued so
        // far (R - 2, fewer near the end) are outstanding; after the barrier
        // every compute wavefront is done with step i - 1, whose slot takes
        // step i + R - 1 while there is one
#pragma unroll
        for (int i = 0; i < KBS; i++) {
            asm volatile("" ::: "memory");
            // (s_waitcnt takes a constant: one case per count, resolved once
            // the loop is unrolled)
            switch (i + R - 2 < KBS ? R - 2 : KBS - 1 - i) {
            case 0: Q4_WAIT_VM_LGKM0(0); break;
            case 1: Q4_WAIT_VM_LGKM0(XI); break;
            case 2: Q4_WAIT_VM_LGKM0(2 * XI); break;
            case 3: Q4_WAIT_VM_LGKM0(3 * XI); break;
            case 4: Q4_WAIT_VM_LGKM0(4 * XI < 63 ? 4 * XI : 63); break;
            case 5: Q4_WAIT_VM_LGKM0(5 * XI < 63 ? 5 * XI : 63); break;
            default: Q4_WAIT_VM_LGKM0(6 * XI < 63 ? 6 * XI : 63); break;
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (i + R - 1 < KBS) issue_x(i + R - 1);
        }
        if (KS > 1) {
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    const int n = blockIdx.x * (16 * NT) + wn * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);
    __builtin_amdgcn_s_barrier();   // the loader's first X slots are issued
    // the k-split group's scales and zero-points as whole runs (the host
    // checks the alignment): 2 NS bytes of scales, NS / 2 bytes of zero-points
    uint32_t sraw[NS / 2], zr[NS / 8];
#pragma unroll
    for (int v = 0; v < NS / 8; v++) zr[v] = 0x88888888u;
    {
        const u32x4 *sp = reinterpret_cast<const u32x4 *>(scales + (nrow * G + (uint32_t)kbase * GPK));
#pragma unroll
        for (int v = 0; v < NS / 8; v++) {
            const u32x4 t = sp[v];
#pragma unroll
            for (int e = 0; e < 4; e++) sraw[4 * v + e] = t[e];
        }
        if (ASYM) {
            const uint8_t *zpp = zeros + (nrow * Gz + ((uint32_t)kbase * GPK >> 1));
            if constexpr (NS >= 32) {
#pragma unroll
                for (int v = 0; v < NS / 32; v++) {
                    const u32x4 t = reinterpret_cast<const u32x4 *>(zpp)[v];
#pragma unroll
                    for (int e = 0; e < 4; e++) zr[4 * v + e] = t[e];
                }
            } else if constexpr (NS == 16) {
                const u32x2 t = *reinterpret_cast<const u32x2 *>(zpp);
                zr[0] = t[0];
                zr[1] = t[1];
            } else {
                zr[0] = *reinterpret_cast<const uint32_t *>(zpp);
            }
        }
    }
    // Code runs: CD k-blocks ahead of the step that uses them. With every run
    // of every wavefront requested at once the runs come back in no useful
    // order and, loads completing in order, a wavefront's first k-block is
    // complete only near the end of the whole stream; a short lead keeps the
    // early k-blocks early.
    u32x4 cw[16];
    auto load_code = [&](int i) {
        cw[i] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)kblock(i) * 64u + q * 16u));
    };
#pragma unroll
    for (int i = 0; i < CD; i++) load_code(i);
    asm volatile("" ::: "memory");

    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Group gi's exact fp32 sums build in part[gi & 1] and are scaled into acc
    // one MFMA step after the group's last one (the products have landed by
    // then). The asm pins each scaling where it stands: left free, the
    // compiler sinks all of them past the loop and keeps every group's
    // partial sums live to the end (hundreds of registers at g = 32).
    floatx4 part[2][MT];
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto scale_group = [&](int gi) {
        const float s = h2f((uint16_t)(sraw[gi >> 1] >> (16 * (gi & 1))));
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int r = 0; r < 4; r++) acc[mt][r] = fmaf(part[gi & 1][mt][r], s, acc[mt][r]);
            asm volatile("" : "+v"(acc[mt]));
        }
    };

    // Step i: the block barrier (the loader has seen slot i land; this
    // wavefront's reads of slot i - 1 are complete), then step i from slot i
    // once the code run of k-block i is in (the compiler's wait).
#pragma unroll
    for (int i = 0; i < KBS; i++) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's LDS reads done
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (i + CD < KBS) load_code(i + CD);
        const unsigned char *slot = ring + (i % R) * SLOT;
        // (1 at 1024, 1/16 at 64) of the zero-point of MFMA step t's group
        auto zadd_of = [&](int t) {
            const int gi = i * GPK + t * GPK / 4;
            const uint32_t zp = (zr[gi >> 3] >> (4 * (gi & 7))) & 15u;
            return (0xE400u + zp) | ((0xD400u + 16u * zp) << 16);
        };
        // at g = 32 / 64 the code dwords of the row's four lane groups are
        // transposed (as in the decode GEMV): MFMA step t then sums the 32-k
        // run t (X chunk 4 t + q), inside one group
        u32x4 w = cw[i];
        if constexpr (GS < 128) {
            const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
            const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
            w = u32x4{s01[0], s01[1], s23[0], s23[1]};
        }
        // all of the step's X fragments first: their LDS latency runs under
        // the unpack instead of in front of each MFMA
        half8 a[4][MT];
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
                a[t][mt] = *reinterpret_cast<const half8 *>(
                    slot + (mt * 16 + r16) * 256 + 16 * ((GS == 128 ? 4 * q + t : 4 * t + q) ^ xswz(r16)));
        // MFMA step t's four products issue with the unpack of step t + 1
        // between them, one pair per product, so the VALU work runs in the
        // matrix core's shadow instead of after it
        u32x4 bv[2];
        {
            const uint32_t z0 = zadd_of(0);
            bv[0] = u32x4{unpack_pair(w[0], 0, z0), unpack_pair(w[0], 1, z0),
                          unpack_pair(w[0], 2, z0), unpack_pair(w[0], 3, z0)};
        }
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const half8 b = __builtin_bit_cast(half8, bv[t & 1]);
            const uint32_t zn = t < 3 ? zadd_of(t + 1) : 0u;
            const int gi = i * GPK + t * GPK / 4;          // the step's group
            const bool first = t % (4 / GPK) == 0;         // its first step
#pragma unroll
            for (int mt = 0; mt < 4; mt++) {
                if (mt < MT)
                    part[gi & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a[t][mt], b, first ? zero4 : part[gi & 1][mt], 0, 0, 0);
                if (t < 3) bv[(t + 1) & 1][mt] = unpack_pair(w[t + 1], mt, zn);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (first && gi > 0) scale_group(gi - 1);
        }
    }
    scale_group(NS - 1);

    if (KS > 1) {
        // the k-split groups' partial sums meet in LDS (group order fixed)
        float *red = reinterpret_cast<float *>(xs);   // [KS - 1][NT wn][MT * 4][64]
        __syncthreads();
        if (ks > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) red[(((ks - 1) * NT + wn) * MT * 4 + mt * 4 + r) * 64 + lane] = acc[mt][r];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; g2++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[mt][r] += red[(((g2 - 1) * NT + wn) * MT * 4 + mt * 4 + r) * 64 + lane];
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = mt * 16 + 4 * q + r;
            if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(acc[mt][r]);
        }
}

// ---------------------------------------------------------------------------
// Batched decode with X resident in LDS (16 rows x K fp16 <= 128 KB: M <= 16
// at K <= 4096). A block of KS x WN wavefronts owns 16 WN output channels;
// wavefront (ks, wn) owns column tile wn over k-split group ks. All of X is
// loaded once (through registers), stored in LDS in the operand k order of
// the decode GEMV's unpack (each 16-byte chunk permuted to k offsets
// 0,4,1,5,2,6,3,7) and XOR-swizzled (chunk c of row m at c ^ xswz(m % 16)); then
// every scale, zero-point and code run of the wavefront's KBW k-blocks is
// issued; one wait and one barrier make X visible, and from there the only
// waits are the compiler's, in issue order, on the code runs. The unpack is
// the GEMV's (9 operations per 8 weights, 16 (u - zp) exact; the 1/16 is
// folded into the fp32 group scale).
template <int WN, int KS, int KBW, bool ASYM, int GS = 128>
__global__ __launch_bounds__(64 * WN * KS) void w4a16_batched_xres_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    static_assert(KS * KBW <= 32, "X must fit the 128 KB of LDS");
    static_assert(GS == 32 || GS == 64 || GS == 128, "group sizes");
    constexpr int GPK = 128 / GS;                 // groups per 128-wide k-block
    constexpr int NS = KBW * GPK;                 // groups of the wavefront's k-blocks
    constexpr int T = 64 * WN * KS;
    __shared__ __attribute__((aligned(1024))) unsigned char xs[32 * 16 * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, ks = wave / WN;    // column tile, k-split group
    const int r16 = lane & 15, q = lane >> 4;
    const int kbase = ks * KBW;
    const int KB = KS * KBW;
    const uint32_t G = (uint32_t)(KB * GPK), Gz = (G + 1) >> 1, kh = (uint32_t)K >> 1;
    const int n = blockIdx.x * 16 * WN + wn * 16 + r16;
    const uint32_t nrow = (uint32_t)(n < N ? n : N - 1);

    // X: 16 B chunk P (= k-block P / 256, row (P / 16) % 16, stored chunk
    // P % 16) at LDS byte 16 P holds logical chunk (P % 16) ^ xswz(row), permuted
    constexpr int NCH = 32 * 16 * 16;                         // chunks when K = 4096
    constexpr int PER = (NCH + T - 1) / T;
    u32x4 xv[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int P = tid + i * T;
        const int kb = P >> 8, m = (P >> 4) & 15, c = (P & 15) ^ xswz(m);
        const int mc = m < M ? m : M - 1;
        xv[i] = u32x4{0u, 0u, 0u, 0u};
        if (kb < KB) xv[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)mc * K + kb * 128 + c * 8);
    }
    // then the scales and zero-points (needed first), then the code runs,
    // after a block barrier: every X load of the block is then ahead of the
    // weight stream in the queues
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    // scales (NS fp16) and zero-points (NS nibbles) of the wavefront's groups
    // as whole vector loads (the host checks the alignment)
    uint32_t sraw[NS / 2], zr[(NS + 7) / 8];
#pragma unroll
    for (int i = 0; i < (NS + 7) / 8; i++) zr[i] = 0x88888888u;
    {
        const uint16_t *sp = scales + (nrow * G + (uint32_t)kbase * GPK);
        if constexpr (NS >= 8) {
#pragma unroll
            for (int v8 = 0; v8 < NS / 8; v8++) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(sp)[v8];
#pragma unroll
                for (int i = 0; i < 4; i++) sraw[4 * v8 + i] = v[i];
            }
        } else if constexpr (NS == 4) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sp);
            sraw[0] = v[0];
            sraw[1] = v[1];
        } else {
            sraw[0] = *reinterpret_cast<const uint32_t *>(sp);
        }
        if (ASYM) {
            const uint8_t *zpp = zeros + (nrow * Gz + ((uint32_t)kbase * GPK >> 1));
            if constexpr (NS == 32) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(zpp);
#pragma unroll
                for (int i = 0; i < 4; i++) zr[i] = v[i];
            } else if constexpr (NS == 16) {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(zpp);
                zr[0] = v[0];
                zr[1] = v[1];
            } else if constexpr (NS == 8) zr[0] = *reinterpret_cast<const uint32_t *>(zpp);
            else if constexpr (NS == 4) zr[0] = *reinterpret_cast<const uint16_t *>(zpp);
            else zr[0] = *zpp;
        }
    }
    asm volatile("" ::: "memory");
    u32x4 cw[KBW];
#pragma unroll
    for (int p = 0; p < KBW; p++)
        cw[p] = *reinterpret_cast<const u32x4 *>(codes + (nrow * kh + (uint32_t)(kbase + p) * 64u + q * 16u));
    // X to LDS in the operand order, then visible to the block
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int P = tid + i * T;
        if ((P >> 8) < KB) *reinterpret_cast<u32x4 *>(xs + P * 16) = permute_x(xv[i]);
    }
    __syncthreads();

    // per k-block: at g = 32 / 64 the four code dwords of the row's four lane
    // groups are transposed first (as in the decode GEMV), so MFMA step t
    // sums one 32-k run (X chunk 4 t + q) inside one group; each group's
    // exact partial sum is scaled by its own scale
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KBW; p++) {
        const unsigned char *slot = xs + (kbase + p) * 4096 + r16 * 256;
        u32x4 w = cw[p];
        if constexpr (GS < 128) {
            const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
            const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
            w = u32x4{s01[0], s01[1], s23[0], s23[1]};
        }
        floatx4 part[GPK];
#pragma unroll
        for (int j = 0; j < GPK; j++) part[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int j = t * GPK / 4, gi = p * GPK + j;
            const ZeroConst zc = zero_const((int)(zr[gi >> 3] >> (4 * (gi & 7))) & 15);
            const int chunk = GS == 128 ? 4 * q + t : 4 * t + q;
            const half8 a = *reinterpret_cast<const half8 *>(slot + 16 * (chunk ^ xswz(r16)));
            part[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, dequant8(w[t], zc), part[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < GPK; j++) {
            const int gi = p * GPK + j;
            const uint32_t sw = sraw[gi >> 1];
            const float s = scale16((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xffffu)));
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(part[j][r], s, acc[r]);
        }
    }

    if (KS > 1) {
        // the k-split groups' partial sums meet in LDS (group order fixed)
        float *red = reinterpret_cast<float *>(xs);   // [KS - 1][WN][4][64]
        __syncthreads();
        if (ks > 0) {
#pragma unroll
            for (int r = 0; r < 4; r++) red[(((ks - 1) * WN + wn) * 4 + r) * 64 + lane] = acc[r];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; g2++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] += red[(((g2 - 1) * WN + wn) * 4 + r) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int m = 4 * q + r;
        if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(acc[r]);
    }
}

// ---------------------------------------------------------------------------
// Batched decode with X in registers (M <= 16, K = 1024 KBW). A block of 8
// wavefronts owns NT column tiles of 16 output channels; wavefront w owns
// k-blocks w KBW .. w KBW + KBW - 1 of all NT tiles. Lane (r16, q) loads the
// X fragments of row r16 over its wavefront's k-range straight into
// registers (64 bytes per k-block; rows >= M stay zero and are not read),
// so a wavefront needs nothing from the others before its first product and
// each X fragment feeds NT tiles' MFMAs. Loads go out as X, then scales and
// zero-points, then the code runs k-block by k-block, all before the first
// wait; each (k-block, tile) is computed once its run has landed. The 8
// partial sums of each output meet in LDS in a fixed order. Unpack and
// arithmetic as in the decode GEMV: 16 (u - zp) exact in fp16, each group's
// exact fp32 partial multiplied by its scale (with the 1/16 folded in). The
// four code dwords of a row are transposed across the lane groups, so MFMA
// step t sums the 32-k run t of the k-block (one group at g = 32, half of
// one at g = 64, a quarter at g = 128) and lane group q's X fragment is
// k = 32 t + 8 q .. + 7: each X load instruction then reads 64 contiguous
// bytes of each of 16 rows.
template <int NT, int KBW, bool ASYM, int GS = 128>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void w4a16_batched_xreg_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ Y)
{
    static_assert(KBW == 2 || KBW == 4, "k-blocks per wavefront");
    static_assert(GS == 32 || GS == 64 || GS == 128, "group sizes");
    constexpr int WV = 8, GPK = 128 / GS, NS = KBW * GPK;   // NS: groups of a wavefront's k-blocks
    __shared__ float red[WV * NT * 4 * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int kb0 = wave * KBW;
    const uint32_t G = (uint32_t)K / GS, Gz = (G + 1) >> 1, kh = (uint32_t)K >> 1;
    const int n0 = (int)blockIdx.x * 16 * NT;

    // 1. X fragments of the wavefront's k-range (zero first, then the load,
    //    so rows >= M need no branch around a pending load)
    u32x4 xa[KBW][4];
#pragma unroll
    for (int p = 0; p < KBW; p++)
#pragma unroll
        for (int t = 0; t < 4; t++) xa[p][t] = u32x4{0u, 0u, 0u, 0u};
    if (r16 < M) {
        const uint16_t *xr = X + ((uint32_t)r16 * (uint32_t)K + (uint32_t)kb0 * 128u);
#pragma unroll
        for (int p = 0; p < KBW; p++)
#pragma unroll
            for (int t = 0; t < 4; t++)
                xa[p][t] = *reinterpret_cast<const u32x4 *>(xr + p * 128 + 32 * t + 8 * q);
    }
    asm volatile("" ::: "memory");
    // 2. scales (NS fp16) and zero-points (NS nibbles) of each tile's row, as
    //    whole vector loads (the host checks the alignment)
    uint32_t nrow[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) {
        const int n = n0 + 16 * j + r16;
        nrow[j] = (uint32_t)(n < N ? n : N - 1);
    }
    uint32_t sraw[NT][NS / 2], zr[NT][(NS + 7) / 8];
#pragma unroll
    for (int j = 0; j < NT; j++) {
#pragma unroll
        for (int i = 0; i < (NS + 7) / 8; i++) zr[j][i] = 0x88888888u;
        const uint16_t *sp = scales + (nrow[j] * G + (uint32_t)kb0 * GPK);
        if constexpr (NS >= 8) {
#pragma unroll
            for (int v8 = 0; v8 < NS / 8; v8++) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(sp)[v8];
#pragma unroll
                for (int i = 0; i < 4; i++) sraw[j][4 * v8 + i] = v[i];
            }
        } else if constexpr (NS == 4) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sp);
            sraw[j][0] = v[0];
            sraw[j][1] = v[1];
        } else {
            sraw[j][0] = *reinterpret_cast<const uint32_t *>(sp);
        }
        if (ASYM) {
            const uint8_t *zpp = zeros + (nrow[j] * Gz + ((uint32_t)kb0 * GPK >> 1));
            if constexpr (NS == 16) {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(zpp);
                zr[j][0] = v[0];
                zr[j][1] = v[1];
            } else if constexpr (NS == 8) zr[j][0] = *reinterpret_cast<const uint32_t *>(zpp);
            else if constexpr (NS == 4) zr[j][0] = *reinterpret_cast<const uint16_t *>(zpp);
            else zr[j][0] = *zpp;
        }
    }
    asm volatile("" ::: "memory");
    // 3. the code runs, k-block by k-block, all issued before the first product
    u32x4 cw[KBW][NT];
#pragma unroll
    for (int p = 0; p < KBW; p++)
#pragma unroll
        for (int j = 0; j < NT; j++)
            cw[p][j] = *reinterpret_cast<const u32x4 *>(codes + (nrow[j] * kh + (uint32_t)(kb0 + p) * 64u + q * 16u));
    // nothing is scheduled across this point: every load above is issued
    // before the first wait for one of them
    __builtin_amdgcn_sched_barrier(0);

    floatx4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KBW; p++) {
        half8 a[4];
#pragma unroll
        for (int t = 0; t < 4; t++) a[t] = __builtin_bit_cast(half8, permute_x(xa[p][t]));
#pragma unroll
        for (int j = 0; j < NT; j++) {
            u32x4 w = cw[p][j];
            {
                const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
                const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
                const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
                const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
                w = u32x4{s01[0], s01[1], s23[0], s23[1]};
            }
            floatx4 part[GPK];
#pragma unroll
            for (int jj = 0; jj < GPK; jj++) part[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int jj = t * GPK / 4, gi = p * GPK + jj;
                const ZeroConst zc = zero_const((int)(zr[j][gi >> 3] >> (4 * (gi & 7))) & 15);
                part[jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], dequant8(w[t], zc), part[jj], 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < GPK; jj++) {
                const int gi = p * GPK + jj;
                const uint32_t sw = sraw[j][gi >> 1];
                const float s = scale16((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xffffu)));
#pragma unroll
                for (int r = 0; r < 4; r++) acc[j][r] = fmaf(part[jj][r], s, acc[j][r]);
            }
        }
    }

    // 4. the wavefronts' partial sums meet in LDS, summed in wavefront order
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) red[((wave * NT + j) * 4 + r) * 64 + lane] = acc[j][r];
    __syncthreads();
    for (int e = (int)threadIdx.x; e < NT * 256; e += WV * 64) {
        const int j = e >> 8, r = (e >> 6) & 3, l = e & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WV; w++) v += red[((w * NT + j) * 4 + r) * 64 + l];
        const int m = 4 * (l >> 4) + r, n = n0 + 16 * j + (l & 15);
        if (m < M && n < N) Y[(int64_t)m * N + n] = f2h(v);
    }
}

// ---------------------------------------------------------------------------
// Large-M GEMM (prefill), M >= 256, g a power of two >= 128. Compute bound.
//
// A block of 8 / WM wavefronts owns a 256 x (32 NU) tile of Y; wavefront w
// owns rows 32 WM w .. 32 WM (w + 1) - 1 of it across all 32 NU columns
// (WM x NU accumulators of v_mfma_f32_32x32x16_f16). K advances 32 at a time.
//   - X never touches LDS: a wavefront's rows are its own, so each lane loads
//     its two 16-byte A fragments of a step straight into registers, two
//     steps ahead.
//   - Thread t owns weight row t of the tile: its 16-byte code run (32
//     nibbles), group scale and zero-point byte come into a four-deep
//     register ring three steps ahead. While the MFMAs of step k run, the
//     thread dequantizes step k + 1's row into one of two LDS buffers as fp16
//     (u - zp) * s, one fp16 pair in the shadow of each column tile.
//   - One barrier per step: after it the dequantized tile of step k is
//     complete and every wavefront is done with the buffer it overwrites.
// LDS rows of the dequantized tile are 64 bytes (4 chunks of 8 k); chunk c
// of row r is stored at c ^ bswz(r), which keeps both the 16-byte operand
// reads and the 16-byte dequant stores conflict-free (below). Every step has the same shape (past the end the last
// step is reloaded), so the loop has no branches and the compiler's waits
// for the register loads stay partial.
//
// Arithmetic. Unlike the decode kernels, the scale is folded into the
// operand: each dequantized weight is f2h((u - zp) * s) with one rounding
// ((u - zp) is exact in fp16 and v_pk_mul_f16 rounds the exact product), so
// one fp32 accumulator serves all groups. The weights' rounding (relative
// <= 2^-11 each) and the fp16 output rounding stay inside the
// 2^-10 * sum |x||w_hat| bound.
constexpr int GBM = 256, GBK = 32;

// Swizzle of the dequantized tile's 64-byte rows: chunk c of row r at
// c ^ bswz(r), bswz(r) = r2 | (r1 ^ r3) << 1 (ri: bit i of r). A fragment
// read (ds_read_b128) takes one chunk of 32 consecutive rows; the gfx950 LDS
// serves it 16 lanes per cycle, four 4-lane groups that share lane bit 5 and
// the parity of lane bits 2-4, 16 bytes of a 256-byte bank row each. A
// dequant store (ds_write_b128) has lane l write row l; it is served 8
// consecutive lanes per cycle over 128 bytes of banks. Both groupings were
// fitted to the bank-conflict counter on probe patterns. Rows 2 apart then
// share a 128-byte slot set, so the store of rows l and l + 2 must differ in
// chunk: with the former c ^ ((r >> 2) & 3) they did not (8 conflict cycles
// per store, none per read); with bswz neither conflicts (measured).
__device__ __forceinline__ int bswz(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }

// fp16 (u - zp) * s of nibbles 2p and 2p + 1 of a code dword, as one fp16
// pair in natural k order. v_perm_b32 copies byte p of w into bytes 0 and 2;
// masking puts the low nibble at bit 0 of the low half (fp16 1024 + u0) and
// the high nibble at bit 4 of the high half (fp16 1024 + 16 u1); one packed
// fma with multipliers (1, 1/16) and addends (-(1024 + zp), -(64 + zp))
// leaves (u0 - zp, u1 - zp) exactly, and one packed multiply by s rounds
// the exact products once.
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, int p, uint32_t zadd, uint32_t s2)
{
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x01010101u * (uint32_t)p);
    const half2v x = __builtin_bit_cast(half2v, and_or(t, 0x00F0000Fu, 0x64006400u));
    const half2v mul = __builtin_bit_cast(half2v, 0x2C003C00u);   // (1, 1/16)
    const half2v v = __builtin_elementwise_fma(x, mul, __builtin_bit_cast(half2v, zadd));
    return __builtin_bit_cast(uint32_t, v * __builtin_bit_cast(half2v, s2));
}

// NF4 form (FMT = kFmtNf4): the codes index the 16 NF4 levels (nf4_dequant8),
// the scales are fp32, one per 64 weights (gshift = 1: two 32-wide steps),
// and each dequantized weight is fp16(level * scale), the exact product
// rounded once. One packed fp16 multiply gives that when
// the scale is an fp16 value, which every scale the NF4 quantizer writes is
// (the max |w| of fp16 weights, or the 1e-8 floor of an all-zero block:
// that rounds to fp16 0, and so does every level * 1e-8, with the level's
// sign either way).
__device__ __forceinline__ u32x4 nf4_scaled8(uint32_t w, float sf)
{
    const u32x4 lv = nf4_dequant8(w);
    const _Float16 h = (_Float16)sf;
    const half2v s2 = {h, h};
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const uint32_t d = lv[p];   // a scalar first: a bit_cast of a vector element reads element 0 here
        r[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, d) * s2);
    }
    return r;
}

// Weight formats of the large-M GEMM: INT4 with group scales (and zero-points),
// NF4 (fp32 scale per 64), NVFP4 (E2M1 codes, E4M3 scale per 16: the two
// scale bytes of a 32-wide step load as the INT4 form's one fp16 scale does,
// gshift = 0, and scale the code dwords 0-1 and 2-3 of the step; e2m1 * e4m3
// is exact in fp16, nvfp4_scaled8).
constexpr int kFmtInt4 = 0, kFmtNf4 = 1, kFmtNvfp4 = 2;

template <int NU, int WM, bool ASYM, int FMT = kFmtInt4>
__global__ __launch_bounds__(512 / WM, 1) void w4a16_gemm_kernel(
    const uint16_t *__restrict__ X, int M, int N, int K, int gshift,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint8_t *__restrict__ zeros, int tiles_m, uint16_t *__restrict__ Y)
{
    constexpr int BN = 32 * NU;
    constexpr int THREADS = 512 / WM;
    static_assert(BN <= THREADS, "one weight row per thread");
    constexpr int B_BYTES = BN * GBK * 2;
    constexpr int B_SPARE = B_BYTES + (THREADS > BN ? THREADS - BN : 0) * 16;
    __shared__ __attribute__((aligned(1024))) unsigned char sb0[B_SPARE];
    __shared__ __attribute__((aligned(1024))) unsigned char sb1[B_SPARE];
    unsigned char *const sb[2] = {sb0, sb1};

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int blocks = gridDim.x, b = blockIdx.x;
    const int t = (blocks % 8 == 0) ? (b % 8) * (blocks / 8) + b / 8 : b;
    const int m0 = (t % tiles_m) * GBM, n0 = (t / tiles_m) * BN;
    const int KT = K / GBK;
    const uint32_t G = (uint32_t)KT >> gshift, Gz = (G + 1) >> 1;

    // this lane's X rows (one per 32-row tile) at k offset 8 h
    uint32_t xoff[WM];
#pragma unroll
    for (int i = 0; i < WM; i++) {
        int m = m0 + wave * 32 * WM + i * 32 + l32;
        m = m < M ? m : M - 1;
        xoff[i] = ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)h) * 2u;
    }
    const unsigned char *Xb = reinterpret_cast<const unsigned char *>(X);
    // this thread's weight row (threads past the tile repeat the last row)
    const int wrow = tid < BN ? tid : BN - 1;
    const uint32_t n_w = (uint32_t)(n0 + wrow < N ? n0 + wrow : N - 1);
    const uint32_t coff = n_w * (uint32_t)(K >> 1), soff = n_w * G, zoff = n_w * Gz;

    u32x4 xa[2][WM][2];   // X fragments, ring of 2 steps
    u32x4 wc[4];          // code runs, ring of 4 steps
    uint32_t ws[4], wz[4];
    auto load_x = [&](int k, int q) {
#pragma unroll
        for (int i = 0; i < WM; i++)
#pragma unroll
            for (int s = 0; s < 2; s++)
                xa[q][i][s] = *reinterpret_cast<const u32x4 *>(Xb + xoff[i] + (uint32_t)k * 64u + 32u * s);
    };
    auto load_w = [&](int k, int q) {
        const uint32_t grp = (uint32_t)k >> gshift;
        wc[q] = *reinterpret_cast<const u32x4 *>(codes + coff + (uint32_t)k * 16u);
        if (FMT == kFmtNf4) ws[q] = reinterpret_cast<const uint32_t *>(scales)[soff + grp];   // fp32 bits
        else ws[q] = scales[soff + grp];
        if (ASYM) wz[q] = zeros[zoff + (grp >> 1)];   // nibble picked at use: no wait here
    };

    floatx16 acc[WM][NU];
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < NU; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int swz = bswz(l32);
    auto read_b = [&](const unsigned char *b_st, int f) {   // f = s * NU + j
        const int s = f / NU, j = f % NU;
        const int co = 16 * ((2 * s + h) ^ swz);
        return *reinterpret_cast<const half8 *>(b_st + (j * 32 + l32) * 64 + co);
    };
    int dq_off = tid * 64, dq_swz = bswz(tid), dq_cs = 16;
    if (BN < THREADS && tid >= BN) {   // all four chunks into the thread's one spare slot
        dq_off = B_BYTES + (tid - BN) * 16;
        dq_swz = 0;
        dq_cs = 0;
    }
    auto wconst = [&](int k, int q, uint32_t &s2, uint32_t &zadd) {
        s2 = (ws[q] & 0xffffu) * 0x10001u;
        const uint32_t zp = ASYM ? (wz[q] >> (4u * (((uint32_t)k >> gshift) & 1u))) & 15u : 8u;
        zadd = (0xE400u + zp) | ((0xD400u + 16u * zp) << 16);   // (-(1024 + zp), -(64 + zp))
    };
    // step k from X slot xq and W buffer u & 1; dequantize W slot (u + 1) & 3
    // (step k + 1) into the other buffer, one pair per column tile
    auto mma_step = [&](int k, int u, int xq) {
        constexpr int F = 2 * NU;
        constexpr int PPF = (16 + F - 1) / F;
        const unsigned char *b_st = sb[u & 1];
        unsigned char *const dq_row = sb[(u + 1) & 1] + dq_off;
        const int wq = (u + 1) & 3;
        uint32_t s2, zadd;
        wconst(k + 1, wq, s2, zadd);
        half8 bq[3];
        bq[0] = read_b(b_st, 0);
        bq[1] = read_b(b_st, 1);
        u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int f = 0; f < F; f++) {
            if (f + 2 < F) bq[(f + 2) % 3] = read_b(b_st, f + 2);
            const int j = f % NU, s = f / NU;
#pragma unroll
            for (int i = 0; i < WM; i++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, xa[xq][i][s]),
                                                                   bq[f % 3], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < PPF; q++) {
                const int pr = f * PPF + q;
                if (pr < 16) {
                    if (FMT == kFmtNf4) {
                        if ((pr & 3) == 0) out = nf4_scaled8(wc[wq][pr >> 2], __builtin_bit_cast(float, ws[wq]));
                    } else if (FMT == kFmtNvfp4) {
                        if ((pr & 3) == 0)
                            out = nvfp4_scaled8(wc[wq][pr >> 2], e4m3_half2((ws[wq] >> (8 * (pr >> 3))) & 0xFFu));
                    } else {
                        out[pr & 3] = dequant_pair(wc[wq][pr >> 2], pr & 3, zadd, s2);
                    }
                    if ((pr & 3) == 3)
                        *reinterpret_cast<u32x4 *>(dq_row + dq_cs * ((pr >> 2) ^ dq_swz)) = out;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt not waited
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // prologue: W of steps 0, 1, 2 and X of steps 0, 1, in the order the
    // loop issues them (so the compiler's wait counts at the loop head agree
    // on both incoming paths); W of step 0 dequantized
    load_w(0, 0);
    load_w(1, 1);
    load_x(0, 0);
    load_w(2 < KT ? 2 : KT - 1, 2);
    load_x(1, 1);
    {
        uint32_t s2, zadd;
        wconst(0, 0, s2, zadd);
        unsigned char *const row = sb[0] + dq_off;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const u32x4 out = FMT == kFmtNf4     ? nf4_scaled8(wc[0][i], __builtin_bit_cast(float, ws[0]))
                              : FMT == kFmtNvfp4 ? nvfp4_scaled8(wc[0][i], e4m3_half2((ws[0] >> (8 * (i >> 1))) & 0xFFu))
                                  : u32x4{dequant_pair(wc[0][i], 0, zadd, s2), dequant_pair(wc[0][i], 1, zadd, s2),
                                          dequant_pair(wc[0][i], 2, zadd, s2), dequant_pair(wc[0][i], 3, zadd, s2)};
            *reinterpret_cast<u32x4 *>(row + dq_cs * (i ^ dq_swz)) = out;
        }
    }
    // Step k (u = k % 4): barrier (W of step k is in its buffer, every
    // wavefront is done with step k - 1); the weights of step k + 3 go to W
    // slot (k + 3) % 4, free since step k - 1's dequant; X of step k + 2 goes
    // to X slot k % 2 once this step's MFMAs have been issued.
    for (int kt = 0; kt < KT; kt += 4) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int k = kt + u;
            barrier();
            load_w(k + 3 < KT ? k + 3 : KT - 1, (u + 3) & 3);
            mma_step(k, u, u & 1);
            load_x(k + 2 < KT ? k + 2 : KT - 1, u & 1);
        }
    }

#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = m0 + wave * 32 * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < NU; j++) {
                const int n = n0 + j * 32 + l32;
                if (n < N) Y[(int64_t)m * N + n] = f2h(acc[i][j][r]);
            }
        }
}

template <int MT, int NT, int PF>
hipError_t launch_skinny(const uint16_t *X, int M, int N, int K, int g, const uint8_t *codes,
                         const uint16_t *scales, const uint8_t *zeros, uint16_t *Y, hipStream_t st)
{
    const int blocks = (N + NT * 16 - 1) / (NT * 16);
    w4a16_skinny_kernel<MT, NT, PF><<<blocks, kThreads, 0, st>>>(X, M, N, K, g, codes, scales,
                                                                 zeros, Y);
    return hipGetLastError();
}

// Group sizes that are not a multiple of 128: the small-group kernel, over
// chunks of at most 65535 block rows.
template <int MT, int NT, int PF>
hipError_t launch_subg_tiles(const uint16_t *X, int64_t M, int N, int K, int g, const uint8_t *codes,
                             const uint16_t *scales, const uint8_t *zeros, uint16_t *Y, hipStream_t st)
{
    constexpr int64_t kRows = 65535LL * MT * 16;
    for (int64_t m0 = 0; m0 < M; m0 += kRows) {
        const int rows = (int)(M - m0 < kRows ? M - m0 : kRows);
        const dim3 grid((unsigned)((N + NT * 16 - 1) / (NT * 16)), (unsigned)((rows + MT * 16 - 1) / (MT * 16)));
        w4a16_subg_kernel<MT, NT, PF><<<grid, kThreads, 0, st>>>(X + m0 * K, rows, N, K, g, codes, scales,
                                                                  zeros, Y + m0 * N);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_subg(const uint16_t *X, int64_t M, int N, int K, int g, const uint8_t *codes,
                       const uint16_t *scales, const uint8_t *zeros, uint16_t *Y, hipStream_t st)
{
    if (M <= 16) return launch_subg_tiles<1, 1, 8>(X, M, N, K, g, codes, scales, zeros, Y, st);
    if (M <= 32) return launch_subg_tiles<2, 2, 4>(X, M, N, K, g, codes, scales, zeros, Y, st);
    return launch_subg_tiles<4, 2, 4>(X, M, N, K, g, codes, scales, zeros, Y, st);
}

// X ring depth of the whole-slice kernel: at most 32 k-blocks of 16 rows in
// the 128 KB, at most 8 slots, and at most 63 loader instructions in flight
// behind the slot a step waits for.
constexpr int cres_ring(int mt, int ks)
{
    const int a = 32 / (mt * ks), b = 2 + 63 / (4 * mt);
    return a < 8 ? (a < b ? a : b) : (8 < b ? 8 : b);
}

// The X-in-registers batched decode for 8 <= M <= 16, K = 2048 or 4096, g =
// 32, 64 or 128, and N <= 4096 (one column tile per block, so at most 256
// blocks, all resident); hipErrorNotSupported otherwise, or when the scale /
// zero-point runs do not suit whole vector loads, or when Q4_XREG=0 (read at
// every call; for A/B measurements). Below 8 rows the decode GEMV (X staged
// in LDS) measured faster; with more column tiles per block (fewer blocks
// for larger N) this kernel measured slower than the X-resident kernel.
hipError_t launch_batched_xreg(const uint16_t *X, int M, int N, int K, int g, const uint8_t *codes,
                               const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                               hipStream_t st)
{
    const char *e = std::getenv("Q4_XREG");
    if ((e && std::atoi(e) == 0) || M < 8 || M > 16 || N > 4096 || (K != 2048 && K != 4096) ||
        (g != 128 && g != 64 && g != 32))
        return hipErrorNotSupported;
    const int kbw = K / 1024, gpk = 128 / g;
    const int G = K / g, Gz = (G + 1) / 2, ns = kbw * gpk;
    const int ssz = 2 * ns < 16 ? 2 * ns : 16, zsz = ns / 2;   // bytes per scale / zero-point load
    if ((reinterpret_cast<uintptr_t>(scales) & (ssz - 1)) != 0 || (2 * G) % ssz != 0 ||
        (zeros && ((reinterpret_cast<uintptr_t>(zeros) & (zsz - 1)) != 0 || Gz % zsz != 0)))
        return hipErrorNotSupported;
    const int blocks = (N + 15) / 16;
    auto go = [&](auto kernel) { kernel<<<blocks, 512, 0, st>>>(X, M, N, K, codes, scales, zeros, Y); };
#define Q4_XREG_A(KBW, GS)                                                                       \
    (zeros ? go(w4a16_batched_xreg_kernel<1, KBW, true, GS>) : go(w4a16_batched_xreg_kernel<1, KBW, false, GS>))
#define Q4_XREG_G(KBW) (g == 128 ? Q4_XREG_A(KBW, 128) : g == 64 ? Q4_XREG_A(KBW, 64) : Q4_XREG_A(KBW, 32))
    if (kbw == 4) Q4_XREG_G(4);
    else Q4_XREG_G(2);
#undef Q4_XREG_G
#undef Q4_XREG_A
    return hipGetLastError();
}

// Batched decode launcher (g = 128 assumed). K is split over KS groups of
// wavefronts inside a block; each group's k-blocks must be a multiple of the
// ring depth.
hipError_t launch_batched(const uint16_t *X, int M, int N, int K, int g, const uint8_t *codes,
                          const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                          hipStream_t st)
{
    if (M < 1 || M > 64 || K % 128 != 0 || (g != 128 && g != 64 && g != 32)) return hipErrorNotSupported;
    const int gpk = 128 / g;
    // these kernels index the codes and X with 32-bit byte offsets; larger
    // operands take the skinny kernel (64-bit offsets)
    if ((int64_t)N * (K / 2) >= ((int64_t)1 << 32) - 256 || (int64_t)M * K * 2 >= ((int64_t)1 << 32))
        return hipErrorNotSupported;
    const int KB = K / 128;
    const int blocks = (N + 63) / 64;
    // X resident in LDS: 16 rows x K fp16 within 128 KB, 4 k-split groups of
    // 2, 4 or 8 k-blocks each, whole-run vector loads of scales / zero-points;
    // 3 column tiles per block when that fills the CUs better than 4
    if (M <= 16 && (KB == 8 || KB == 16 || KB == 32)) {
        const int kbw = KB / 4;
        // a wavefront's ns groups: scales in loads of up to 16 bytes, zero-points
        // in one load of ns / 2 bytes; every row of both must start on them
        const int G = KB * gpk, Gz = (G + 1) / 2, ns = kbw * gpk;
        const int ssz = 2 * ns < 16 ? 2 * ns : 16, zsz = ns / 2;
        const bool aligned = (reinterpret_cast<uintptr_t>(scales) & (ssz - 1)) == 0 && (2 * G) % ssz == 0 &&
                             (!zeros || ((reinterpret_cast<uintptr_t>(zeros) & (zsz - 1)) == 0 &&
                                         Gz % zsz == 0));
        if (aligned) {
            const int b4 = (N + 63) / 64, b3 = (N + 47) / 48;
            const bool three = b3 <= 256 && b4 < 256;   // every CU busy with 3, some idle with 4
            const int nb = three ? b3 : b4;
            auto go = [&](auto kernel, int wn) { kernel<<<nb, 256 * wn, 0, st>>>(X, M, N, K, codes, scales, zeros, Y); };
#define Q4_XRES_G(WN, GS)                                                                             \
    do {                                                                                              \
        if (kbw == 8) zeros ? go(w4a16_batched_xres_kernel<WN, 4, 8, true, GS>, WN) : go(w4a16_batched_xres_kernel<WN, 4, 8, false, GS>, WN); \
        else if (kbw == 4) zeros ? go(w4a16_batched_xres_kernel<WN, 4, 4, true, GS>, WN) : go(w4a16_batched_xres_kernel<WN, 4, 4, false, GS>, WN); \
        else zeros ? go(w4a16_batched_xres_kernel<WN, 4, 2, true, GS>, WN) : go(w4a16_batched_xres_kernel<WN, 4, 2, false, GS>, WN); \
    } while (0)
#define Q4_XRES(WN)                                                                                   \
    do {                                                                                              \
        if (g == 128) Q4_XRES_G(WN, 128);                                                             \
        else if (g == 64) Q4_XRES_G(WN, 64);                                                          \
        else Q4_XRES_G(WN, 32);                                                                       \
    } while (0)
            if (three) Q4_XRES(3);
            else Q4_XRES(4);
#undef Q4_XRES
#undef Q4_XRES_G
            return hipGetLastError();
        }
    }
    auto launch = [&](auto kernel, int ks) {
        kernel<<<blocks, 256 * ks, 0, st>>>(X, M, N, K, codes, scales, zeros, Y);
    };
    // the whole-slice kernel: NT compute wavefronts (NT column tiles) and one
    // X loader per k-split group; 3 column tiles when that still makes at most
    // one round of blocks and 4 would leave CUs idle
    const int cb3 = (N + 47) / 48, cb4 = (N + 63) / 64;
    const bool nt3 = cb3 <= 256 && cb4 < 256;
    auto launch_cres = [&](auto kernel, int ks, int nt) {
        kernel<<<nt == 3 ? cb3 : cb4, 64 * (nt + 1) * ks, 0, st>>>(X, M, N, K, codes, scales, zeros, Y);
    };
    // M > 16 with at most 16 k-blocks per k-split group: the wavefront's
    // weight slice is held in registers, only X goes through the LDS ring
    // (8 slots, or 4 when 4 m-tiles and 2 groups share the 128 KB)
    // (scales: whole 16-byte runs; zero-points: runs of KBS gpk / 2 bytes, at
    // most 16 per load; every row of both arrays holds whole runs for these K)
    const int kbs_z = (KB == 32 ? 16 : 8) * gpk / 2;
    const bool runs_aligned = (reinterpret_cast<uintptr_t>(scales) & 15) == 0 &&
                              (!zeros || (reinterpret_cast<uintptr_t>(zeros) & ((kbs_z < 16 ? kbs_z : 16) - 1)) == 0);
    if (M > 16 && (KB == 8 || KB == 16 || KB == 32) && runs_aligned) {
#define Q4_C_G(MT, KS, KBS, GS)                                                                                    \
    (zeros ? (nt3 ? launch_cres(w4a16_batched_cres_kernel<MT, KS, cres_ring(MT, KS), KBS, true, 3, GS>, KS, 3)     \
                  : launch_cres(w4a16_batched_cres_kernel<MT, KS, cres_ring(MT, KS), KBS, true, 4, GS>, KS, 4))    \
           : (nt3 ? launch_cres(w4a16_batched_cres_kernel<MT, KS, cres_ring(MT, KS), KBS, false, 3, GS>, KS, 3)    \
                  : launch_cres(w4a16_batched_cres_kernel<MT, KS, cres_ring(MT, KS), KBS, false, 4, GS>, KS, 4)))
#define Q4_C(MT, KS, KBS)                                                                                          \
    (g == 128 ? Q4_C_G(MT, KS, KBS, 128) : g == 64 ? Q4_C_G(MT, KS, KBS, 64) : Q4_C_G(MT, KS, KBS, 32))
        const bool mt2 = M <= 32;
        if (KB == 32) mt2 ? Q4_C(2, 2, 16) : Q4_C(4, 2, 16);
        else if (KB == 16) mt2 ? Q4_C(2, 2, 8) : Q4_C(4, 2, 8);
        else mt2 ? Q4_C(2, 1, 8) : Q4_C(4, 1, 8);
#undef Q4_C
#undef Q4_C_G
        return hipGetLastError();
    }
    if (g != 128) return hipErrorNotSupported;   // the ring kernel below sums whole 128-wide groups
#define Q4_B(MT, KS)                                                                        \
    (zeros ? launch(w4a16_batched_kernel<MT, KS, 4, 4, true>, KS)                           \
           : launch(w4a16_batched_kernel<MT, KS, 4, 4, false>, KS))
    // X ring and code ring equally deep (4): loads complete in order, so a
    // deeper code ring would only wait behind the X slots anyway
    if (M <= 16) {   // 16 wavefronts: four k-split groups
        if (KB % 16 == 0) Q4_B(1, 4);
        else return hipErrorNotSupported;
    } else {         // 8 wavefronts: two k-split groups
        if (KB % 8 != 0) return hipErrorNotSupported;
        if (M <= 32) Q4_B(2, 2);
        else Q4_B(4, 2);
    }
#undef Q4_B
    return hipGetLastError();
}

}  // namespace

namespace {

// The lookup-decoded formats on the large-M GEMM (symmetric, no zero-points):
// the INT4 form's tile width rule, FMT's B-fragment producer.
template <int FMT>
hipError_t launch_lut_gemm(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                           const uint16_t *sc, int gshift, uint16_t *Y, hipStream_t st)
{
    if (M < 1 || N < 1 || K % 128 != 0 || M * K * 2 >= ((int64_t)1 << 31) || N * (K / 2) >= ((int64_t)1 << 31))
        return hipErrorNotSupported;
    const int m = (int)M, n = (int)N, k = (int)K;
    const int tiles_m = (m + GBM - 1) / GBM;
    int best = gemm_nu_override();
    if (best == 0) {   // the tile width rule of launch_w4a16
        int64_t best_cost = 0;
        const int nus[3] = {4, 8, 11};
        for (int c = 0; c < 3; c++) {
            const int64_t tiles = (int64_t)tiles_m * ((n + 32 * nus[c] - 1) / (32 * nus[c]));
            const int64_t cost = (tiles + 255) / 256 * (nus[c] + 2);
            if (best == 0 || cost < best_cost) { best = nus[c]; best_cost = cost; }
        }
    }
    const int tiles = tiles_m * ((n + 32 * best - 1) / (32 * best));
    auto launch = [&](auto kernel, int threads) {
        kernel<<<tiles, threads, 0, st>>>(X, m, n, k, gshift, codes, sc, nullptr, tiles_m, Y);
    };
    if (best == 4) launch(w4a16_gemm_kernel<4, 2, false, FMT>, 256);
    else if (best == 8) launch(w4a16_gemm_kernel<8, 2, false, FMT>, 256);
    else launch(w4a16_gemm_kernel<11, 1, false, FMT>, 512);
    return hipGetLastError();
}

}  // namespace

// NF4: fp32 scales, one per 64 = two 32-wide steps (gshift 1)
hipError_t launch_nf4_gemm(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                          const float *scales, uint16_t *Y, hipStream_t st)
{
    return launch_lut_gemm<kFmtNf4>(X, M, N, K, codes, reinterpret_cast<const uint16_t *>(scales), 1, Y, st);
}

// NVFP4: two E4M3 scale bytes per 32-wide step, read as one 16-bit unit (gshift 0)
hipError_t launch_nvfp4_gemm(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                            const uint8_t *scales, uint16_t *Y, hipStream_t st)
{
    return launch_lut_gemm<kFmtNvfp4>(X, M, N, K, codes, reinterpret_cast<const uint16_t *>(scales), 0, Y, st);
}

hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                        const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        uint16_t *Y, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    const int m = (int)M, n = (int)N, k = (int)K;
    if ((g == 128 || g == 64 || g == 32) && M >= 8 && M <= 16) {
        const hipError_t e = launch_batched_xreg(X, m, n, k, g, codes, scales, zeros, Y, st);
        if (e != hipErrorNotSupported) return e;
    }
    if ((g == 128 || g == 64 || g == 32) && M <= 16) {
        const hipError_t e = launch_w4a16_gemv(X, M, N, K, g, codes, scales, zeros, Y, st);
        if (e != hipErrorNotSupported) return e;
    }
    if (M >= 256 && g % 32 == 0 && (g & (g - 1)) == 0 && K % 128 == 0 &&
        M * K * 2 < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31)) {
        // Tile width 32 NU: one block per CU, so the time is about the number
        // of full-chip rounds of 256 tiles times (tile width + a fixed
        // per-tile cost of ~2 units for pipeline fill and the epilogue).
        int best = gemm_nu_override();
        const int tiles_m = (m + GBM - 1) / GBM;
        if (best == 0) {
            int64_t best_cost = 0;
            const int nus[3] = {4, 8, 11};
            for (int c = 0; c < 3; c++) {
                const int64_t tiles = (int64_t)tiles_m * ((n + 32 * nus[c] - 1) / (32 * nus[c]));
                const int64_t cost = (tiles + 255) / 256 * (nus[c] + 2);
                if (best == 0 || cost < best_cost) { best = nus[c]; best_cost = cost; }
            }
        }
        const int tiles = tiles_m * ((n + 32 * best - 1) / (32 * best));
        const int gshift = __builtin_ctz((unsigned)(g / GBK));
        auto launch = [&](auto kernel, int threads) {
            kernel<<<tiles, threads, 0, st>>>(X, m, n, k, gshift, codes, scales, zeros, tiles_m, Y);
        };
        const bool asym = zeros != nullptr;
        if (best == 4) asym ? launch(w4a16_gemm_kernel<4, 2, true>, 256) : launch(w4a16_gemm_kernel<4, 2, false>, 256);
        else if (best == 8) asym ? launch(w4a16_gemm_kernel<8, 2, true>, 256) : launch(w4a16_gemm_kernel<8, 2, false>, 256);
        else asym ? launch(w4a16_gemm_kernel<11, 1, true>, 512) : launch(w4a16_gemm_kernel<11, 1, false>, 512);
        return hipGetLastError();
    }
    if ((g == 128 || g == 64 || g == 32) && M <= 64) {
        const hipError_t e = launch_batched(X, m, n, k, g, codes, scales, zeros, Y, st);
        if (e != hipErrorNotSupported) return e;
    }
    if (g % 128 != 0) return launch_subg(X, M, n, k, g, codes, scales, zeros, Y, st);
    if (M <= 16) return launch_skinny<1, 1, 8>(X, m, n, k, g, codes, scales, zeros, Y, st);
    if (M <= 32) return launch_skinny<2, 2, 4>(X, m, n, k, g, codes, scales, zeros, Y, st);
    if (M <= 64) return launch_skinny<4, 2, 4>(X, m, n, k, g, codes, scales, zeros, Y, st);
    dim3 grid((unsigned)((N + PBN - 1) / PBN), (unsigned)((M + PBM - 1) / PBM));
    w4a16_prefill_kernel<<<grid, kThreads, 0, st>>>(X, m, n, k, g, codes, scales, zeros, Y);
    return hipGetLastError();
}

}  // namespace q4k
