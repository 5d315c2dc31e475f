// W8A8 INT8 GEMM on gfx950 with exact int32 accumulation and the scale
// epilogue (Quantization operators guide, blog.freezetheflame.cc, §2.3: the
// int32 accumulator dequantized in the GEMM epilogue as acc * scale_A *
// scale_B; §5.2 path A: the smoothing factor is already inside the weight
// scale, so the epilogue needs only the per-token and per-channel scales).
//
// Both operands are K-contiguous ([M, K] and [N, K]), so every lane loads 16
// consecutive int8 along K: exactly one v_mfma_i32_16x16x64_i8 operand. As in
// the fp16 kernels, A and B see the same k order inside an MFMA, which makes
// the choice of order free; here lane group q takes bytes [16q, 16q + 16) of
// each 64-wide k-step.
//
// Built with -ffp-contract=off: the epilogue is ((float)acc * sx) * sw, two
// fp32 roundings then one fp16 rounding, the same expression as the pages'.
#include "q4_internal.hpp"

namespace q4k {
namespace {

constexpr int kThreads = 256;
constexpr int QBM = 128, QBN = 128, QBK = 128, QLD = QBK + 16;   // LDS row stride in bytes

// A 256-thread block computes a 128 x 128 tile; 4 wavefronts in a 2 x 2 grid
// of 64 x 64 sub-tiles (4 x 4 MFMA tiles of 16 x 16, 64 int32 accumulators per
// lane). K advances 128 bytes per step: tiles are loaded into registers one
// step ahead and staged through LDS.
__global__ __launch_bounds__(kThreads, 2) void w8a8_gemm_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    __shared__ __attribute__((aligned(16))) int8_t Xs[QBM][QLD];
    __shared__ __attribute__((aligned(16))) int8_t Ws[QBN][QLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.y * QBM, n0 = blockIdx.x * QBN;
    const int KT = (K + QBK - 1) / QBK;

    const int lc = tid & 7, lr0 = tid >> 3;   // 8 chunks of 16 bytes per row, 4 rows/thread
    u32x4 xreg[4], wreg[4];

    auto load_tile = [&](int kt) {
        const int k = kt * QBK + lc * 16;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + lr0 + 32 * i;
            const int n = n0 + lr0 + 32 * i;
            xreg[i] = u32x4{0u, 0u, 0u, 0u};
            wreg[i] = u32x4{0u, 0u, 0u, 0u};
            if (k < K) {
                if (m < M) xreg[i] = *reinterpret_cast<const u32x4 *>(Xq + (int64_t)m * K + k);
                if (n < N) wreg[i] = *reinterpret_cast<const u32x4 *>(Wq + (int64_t)n * K + k);
            }
        }
    };

    intx4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 4; nt++) acc[mt][nt] = intx4{0, 0, 0, 0};

    load_tile(0);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; i++) {
            *reinterpret_cast<u32x4 *>(&Xs[lr0 + 32 * i][lc * 16]) = xreg[i];
            *reinterpret_cast<u32x4 *>(&Ws[lr0 + 32 * i][lc * 16]) = wreg[i];
        }
        __syncthreads();
        if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
        for (int s = 0; s < QBK / 64; s++) {
            intx4 a[4], b[4];
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
                a[mt] = *reinterpret_cast<const intx4 *>(&Xs[wm * 64 + mt * 16 + r16][s * 64 + q * 16]);
#pragma unroll
            for (int nt = 0; nt < 4; nt++)
                b[nt] = *reinterpret_cast<const intx4 *>(&Ws[wn * 64 + nt * 16 + r16][s * 64 + q * 16]);
#pragma unroll
            for (int mt = 0; mt < 4; mt++)
#pragma unroll
                for (int nt = 0; nt < 4; nt++)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], b[nt], acc[mt][nt],
                                                                         0, 0, 0);
        }
    }

#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = m0 + wm * 64 + mt * 16 + 4 * q + r;
            if (m >= M) continue;
            const float xs = sx[m];
#pragma unroll
            for (int nt = 0; nt < 4; nt++) {
                const int n = n0 + wn * 64 + nt * 16 + r16;
                if (n >= N) continue;
                const int32_t a = acc[mt][nt][r];
                if (acc_out) acc_out[(int64_t)m * N + n] = a;
                float f = (float)a * xs;
                f = f * sw[n];
                // Keep the fp32 product: without this the backend folds the
                // multiply and the fp16 convert into one v_fma_mix (a single
                // rounding), which differs from fp32-then-fp16 on rare ties.
                asm volatile("" : "+v"(f));
                Y[(int64_t)m * N + n] = f2h(f);
            }
        }
}

}  // namespace

hipError_t launch_w8a8_gemm(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                            int64_t M, int64_t N, int64_t K, uint16_t *Y, int32_t *acc_out,
                            hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + QBN - 1) / QBN), (unsigned)((M + QBM - 1) / QBM));
    w8a8_gemm_kernel<<<grid, kThreads, 0, st>>>(Xq, sx, Wq, sw, (int)M, (int)N, (int)K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace q4k
