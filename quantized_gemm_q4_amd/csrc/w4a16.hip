// W4A16 linear layer on gfx950: Y[M,N] = X[M,K] * W_hat[N,K]^T with the INT4
// weight dequantized inside the GEMM (Quantization operators guide,
// blog.freezetheflame.cc, §1.2: quantize / compute / dequantize fused into
// the GEMM; Core ideas, ai-infra.cypggs.com, §2.2: w_hat = (u - zp) * s;
// Method boundaries, llm-glossary.tokens-kit.com, GPTQ section: decode is
// bound by the weight read, prefill by the dequant + matrix-core path).
//
// Arithmetic. Both kernels feed v_mfma_f32_16x16x32_f16 with the exact
// integers (u - zp) in fp16 and x in fp16: every product is exact in fp32.
// The fp32 partial sum of one 128-wide k-block is multiplied by the fp32
// value of the block's group scale and added to the fp32 total. The only
// roundings are fp32 additions and the final fp16 store.
//
// Operand layout. In a 16x16x32 MFMA lane l feeds row (l % 16) of A and column
// (l % 16) of B with 8 k-values each; A and B see the same k order, so the
// product does not depend on which k sits where. We pick the order that makes
// the INT4 unpack cheap: lane group q = l / 16 owns the 32 consecutive k of
// a 128-wide k-block starting at 32q (one 16-byte load of codes), and
// MFMA step t takes the 8 nibbles of the lane's dword t. The mask
// (w >> 4i) & 0x000F000F lifts nibbles i and i+4 into the two fp16 halves of
// a register at once, so the B operand holds k offsets (0,4,1,5,2,6,3,7);
// the X operand is permuted the same way.
//
// The packed weight is read in place in the layout q4_quantize_pack writes
// (row-major codes [N, K/2], scales [N, K/g], zeros [N, ceil(K/g/2)]); it is
// never expanded in memory.
#include "q4_internal.hpp"

namespace q4k {
namespace {

constexpr int kThreads = 256;

// fp16 pair (1024 + nib_i, 1024 + nib_{i+4}) for i = 0..3 minus (1024 + zp):
// exact small integers. zb holds the fp16 pair (1024 + zp, 1024 + zp).
__device__ __forceinline__ half8 dequant8(uint32_t w, uint32_t zb)
{
    const uint32_t mask = 0x000F000Fu, magic = 0x64006400u;   // fp16 1024.0
    const half2v z = __builtin_bit_cast(half2v, zb);
    const half2v p0 = __builtin_bit_cast(half2v, (w & mask) | magic) - z;
    const half2v p1 = __builtin_bit_cast(half2v, ((w >> 4) & mask) | magic) - z;
    const half2v p2 = __builtin_bit_cast(half2v, ((w >> 8) & mask) | magic) - z;
    const half2v p3 = __builtin_bit_cast(half2v, ((w >> 12) & mask) | magic) - z;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ uint32_t zero_pair(int zp)
{
    return (uint32_t)(0x6400 + zp) * 0x10001u;
}

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
        uint32_t zb[PF][NT];
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int kb = kb0 + p;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                if (kb < kb_end) {
                    const int grp = kb / bpg;
                    cw[p][nt] = *reinterpret_cast<const u32x4 *>(codes + nrow[nt] * row_bytes +
                                                                 kb * 64 + q * 16);
                    sc[p][nt] = h2f(scales[nrow[nt] * G + grp]);
                    zb[p][nt] = zero_pair(group_zp(zeros, nrow[nt], Gz, grp));
                } else {
                    cw[p][nt] = u32x4{0u, 0u, 0u, 0u};
                    sc[p][nt] = 0.0f;
                    zb[p][nt] = zero_pair(0);
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
    uint32_t zreg[2];
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
            zreg[i] = zero_pair(group_zp(zeros, n, Gz, grp));
        }
        if (tid < PBN) {
            int n = n0 + tid;
            n = n < N ? n : N - 1;
            sreg = h2f(scales[(int64_t)n * G + grp]);
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

template <int MT, int NT, int PF>
hipError_t launch_skinny(const uint16_t *X, int M, int N, int K, int g, const uint8_t *codes,
                         const uint16_t *scales, const uint8_t *zeros, uint16_t *Y, hipStream_t st)
{
    const int blocks = (N + NT * 16 - 1) / (NT * 16);
    w4a16_skinny_kernel<MT, NT, PF><<<blocks, kThreads, 0, st>>>(X, M, N, K, g, codes, scales,
                                                                 zeros, Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                        const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        uint16_t *Y, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    const int m = (int)M, n = (int)N, k = (int)K;
    if (M <= 16) return launch_skinny<1, 1, 8>(X, m, n, k, g, codes, scales, zeros, Y, st);
    if (M <= 32) return launch_skinny<2, 2, 4>(X, m, n, k, g, codes, scales, zeros, Y, st);
    if (M <= 64) return launch_skinny<4, 2, 4>(X, m, n, k, g, codes, scales, zeros, Y, st);
    dim3 grid((unsigned)((N + PBN - 1) / PBN), (unsigned)((M + PBM - 1) / PBM));
    w4a16_prefill_kernel<<<grid, kThreads, 0, st>>>(X, m, n, k, g, codes, scales, zeros, Y);
    return hipGetLastError();
}

}  // namespace q4k
