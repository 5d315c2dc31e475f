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
#include <type_traits>

#include <cstdlib>
#include <cstring>

#include "q4_internal.hpp"
#include "row_codes.hpp"

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

// ---------------------------------------------------------------------------
// Large-tile kernel (K % 128 == 0). Built around v_mfma_i32_32x32x32_i8, which
// runs near the int8 peak on gfx950 where the 16x16x64 form does not. A
// 512-thread block computes a 256 x 256 tile of Y; its 8 wavefronts form a
// 2 (M) x 4 (N) grid of 128 x 64 sub-tiles (4 x 2 MFMA tiles of 32 x 32, 128
// int32 accumulators per lane).
//
// Operand staging: K advances 64 bytes per step through five LDS stages
// (32 KB each: 256 rows of X and 256 rows of W, 64 bytes per row; the five
// fill the 160 KB of LDS), filled by direct global-to-LDS loads
// (global_load_lds_dwordx4, lane i of a load lands at base + 16 i) issued
// four steps ahead, so a step's data has four steps of MFMA work to arrive
// in and no registers are spent on staging. Before a stage is read every
// wavefront waits for its own loads of that stage (vmcnt) and for its
// earlier LDS reads (lgkmcnt), then the block meets at a barrier. The
// 16-byte chunks of a row are stored XOR-swizzled (chunk c of row r at
// c ^ ((r >> 2) & 3)) so the 32 rows an operand read touches fall in
// distinct banks.
//
// Output layout: the MFMAs take W as their first operand and X as their
// second, so each 32 x 32 accumulator tile is a tile of Y transposed: lane l
// holds row l % 32 of Y and columns 8 (r / 4) + 4 (l / 32) + r % 4, i.e. four
// consecutive outputs of one row per group of four registers. The epilogue
// needs one per-token scale per 32-row tile and writes each group as one
// 8-byte LDS store; the block's 256 x 256 fp16 tile is staged in the (then
// free) LDS and written back as whole rows with 16-byte stores.
//
// Tile order is XCD-aware: consecutive block ids go to the 8 XCDs in turn, so
// block b computes tile t = (b % 8) * (blocks / 8) + b / 8; each XCD then owns
// whole columns of N-tiles, and its L2 serves their reuse of the W tiles.
constexpr int LBM = 256, LBN = 256, LBK = 64, LSTAGES = 5;
constexpr int LSTAGE_BYTES = (LBM + LBN) * LBK;   // 32 KB
constexpr int OUT_STRIDE = LBN * 2 + 16;            // bytes per row of the staged fp16 output tile
constexpr int LDS_BYTES = LBM * OUT_STRIDE > LSTAGES * LSTAGE_BYTES ? LBM * OUT_STRIDE : LSTAGES * LSTAGE_BYTES;


// The same kernel serves FP8 E4M3 operands (FP8 = true; Quantization
// operators guide §4.2: C = scale_A scale_B (A_fp8 @ B_fp8)): each 64-byte
// step is then one v_mfma_f32_32x32x64_f8f6f4 per 32 x 32 tile (both k32
// halves' fragments side by side: A and B agree on the k order, so the sum
// is the same), with fp32 accumulators; the first half of a step's MFMAs is
// tiles i = 0, 1, the second i = 2, 3. No int32 output in that form.
template <bool FP8>
__global__ __launch_bounds__(512, 1) void w8a8_gemm_large_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int M, int N, int K, int tiles_m, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    using Acc = typename std::conditional<FP8, floatx16, intx16>::type;
    __shared__ __attribute__((aligned(1024))) int8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, h = lane >> 5;

    const int blocks = gridDim.x;
    const int b = blockIdx.x;
    const int t = (blocks % 8 == 0) ? (b % 8) * (blocks / 8) + b / 8 : b;
    const int m0 = (t % tiles_m) * LBM, n0 = (t / tiles_m) * LBN;
    const int KT = K / LBK;

    // Direct-load assignment: a stage holds 32 blocks of 1 KB (16 rows x 64 B):
    // blocks 0-15 are X rows, 16-31 W rows; wavefront w loads blocks 2w, 2w+1
    // (X) and 16 + 2w, 16 + 2w + 1 (W). Lane i of block q writes row
    // 16 q + i / 4, stored chunk i % 4, which holds logical chunk
    // (i % 4) ^ ((i >> 4) & 3).
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t goff[4];                    // byte offsets from Xq (j < 2) or Wq (j >= 2)
#pragma unroll
    for (int j = 0; j < 2; j++) {
        int m = m0 + (2 * wave + j) * 16 + (lane >> 2);
        int n = n0 + (2 * wave + j) * 16 + (lane >> 2);
        m = m < M ? m : M - 1;
        n = n < N ? n : N - 1;
        goff[j] = (uint32_t)m * (uint32_t)K + 16 * dchunk;
        goff[2 + j] = (uint32_t)n * (uint32_t)K + 16 * dchunk;
    }
    auto issue = [&](int8_t *stage, int kt) {
        const uint32_t kofs = (uint32_t)kt * LBK;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            __builtin_amdgcn_global_load_lds(Xq + goff[j] + kofs, stage + (2 * wave + j) * 1024, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(Wq + goff[2 + j] + kofs,
                                             stage + (16 + 2 * wave + j) * 1024, 16, 0, 0);
        }
    };

    // operand read offsets inside a stage (swizzled chunk per k32 step s)
    const int swz = (l32 >> 2) & 3;
    const int co0 = 16 * ((0 + h) ^ swz), co1 = 16 * ((2 + h) ^ swz);
    const int arow = (wm * 128 + l32) * LBK;
    const int brow = LBM * LBK + (wn * 64 + l32) * LBK;

    Acc acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    // Operand fragments of one 64-byte step: both k32 halves are read before
    // the first MFMA, so the second half's LDS latency hides under the first
    // half's MFMAs.
    struct Frags {
        intx4 a[2][4], b[2][2];
    };
    auto read = [&](const int8_t *stage, Frags &f) {
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const int co = s ? co1 : co0;
#pragma unroll
            for (int i = 0; i < 4; i++)
                f.a[s][i] = *reinterpret_cast<const intx4 *>(stage + arow + i * 32 * LBK + co);
#pragma unroll
            for (int j = 0; j < 2; j++)
                f.b[s][j] = *reinterpret_cast<const intx4 *>(stage + brow + j * 32 * LBK + co);
        }
    };
    auto mma_half = [&](const Frags &f, int s) {   // the first or second half of a step's MFMAs
        if constexpr (FP8) {
#pragma unroll
            for (int i = 2 * s; i < 2 * s + 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const intx8 a = __builtin_shufflevector(f.a[0][i], f.a[1][i], 0, 1, 2, 3, 4, 5, 6, 7);
                    const intx8 bb = __builtin_shufflevector(f.b[0][j], f.b[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
                    // format 0 = E4M3 for both operands; scale operands 0 select the unscaled form
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bb, a, acc[i][j], 0, 0, 0, 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[s][j], f.a[s][i], acc[i][j], 0, 0, 0);
        }
    };

    // Software pipeline (five LDS stages, two register fragment sets). Step
    // k: run the first half of step k's MFMAs from registers, wait for this
    // wavefront's loads of stage k + 1 and meet the block at the barrier
    // (after it stage k + 1 is complete and everyone is done reading stage
    // k), then interleave the second half of the MFMAs with the reads of
    // stage k + 1's fragments and the refill of stage k with step k + 5, so
    // the matrix pipe never waits on the barrier's LDS and load traffic.
    // Every step has the same shape: past the end the last step is
    // refetched into stages nobody reads, so the wait counts are uniform.
#pragma unroll
    for (int p = 0; p < LSTAGES; p++) issue(lds + p * LSTAGE_BYTES, p < KT ? p : KT - 1);
    Frags f[2];
    asm volatile("" ::: "memory");
    Q4_WAIT_VM_LGKM0(4 * (LSTAGES - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read(lds, f[0]);
    int sc = 0;   // stage of step k (k mod 5)
    for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int k = kt + u;
            const int sn = sc == LSTAGES - 1 ? 0 : sc + 1;
            mma_half(f[u], 0);
            // nothing may move across the barrier (the scheduler does not
            // treat s_barrier as a boundary for LDS reads by itself)
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            Q4_WAIT_VM_LGKM0(4 * (LSTAGES - 2));   // loads outstanding: stages k + 2 .. k + 4
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            read(lds + sn * LSTAGE_BYTES, f[u ^ 1]);
            issue(lds + sc * LSTAGE_BYTES, k + LSTAGES < KT ? k + LSTAGES : KT - 1);
            mma_half(f[u], 1);
            if constexpr (FP8) {
                // 12 fragment reads and 4 loads between the 4 MFMAs
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (g >= 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // VMEM read
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);               // DS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
                }
            } else {
                // 12 fragment reads and 4 loads between the 8 MFMAs
#pragma unroll
                for (int g = 0; g < 6; g++) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                }
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);       // VMEM read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            sc = sn;
        }
    }
    Q4_WAIT_VM_LGKM0(0);   // the refetches past the end
    // lane's outputs: row wm * 128 + 32 i + l32 of the block tile, columns
    // wn * 64 + 32 j + 8 q + 4 h + e for accumulator r = 4 q + e
    if constexpr (!FP8) {
    if (acc_out) {
        const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(acc_out) & 15) == 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + wm * 128 + i * 32 + l32;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int n = n0 + wn * 64 + j * 32 + 8 * q + 4 * h;
                    int32_t *const dst = acc_out + (int64_t)m * N + n;
                    if (vec_ok && n + 4 <= N) {
                        *reinterpret_cast<intx4 *>(dst) =
                            intx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (n + e < N) dst[e] = acc[i][j][4 * q + e];
                    }
                }
        }
    }
    }
    // Epilogue: y = f2h((acc * sx[m]) * sw[n]), staged through LDS as the
    // block's 256 x 256 fp16 tile, then written back as whole rows with
    // 16-byte stores.
    // All 36 scale loads of a lane go out at once, so the epilogue pays one
    // memory latency rather than one per column group.
    float xsv[4], swv[2][4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = m0 + wm * 128 + i * 32 + l32;
        xsv[i] = sx[m < M ? m : M - 1];
    }
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int n = n0 + wn * 64 + j * 32 + 8 * q + 4 * h + e;
                swv[j][q][e] = sw[n < N ? n : N - 1];
            }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();   // every wavefront is done with the stages
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int nl = wn * 64 + j * 32 + 8 * q + 4 * h;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t pk[2];
#pragma unroll
                for (int e2 = 0; e2 < 2; e2++) {
                    uint32_t hv[2];
#pragma unroll
                    for (int e1 = 0; e1 < 2; e1++) {
                        const int e = 2 * e2 + e1;
                        float f = (float)acc[i][j][4 * q + e] * xsv[i];
                        f = f * swv[j][q][e];
                        // Keep the fp32 product: without this the backend
                        // folds the multiply and the fp16 convert into one
                        // v_fma_mix (a single rounding).
                        asm volatile("" : "+v"(f));
                        hv[e1] = f2h(f);
                    }
                    pk[e2] = hv[0] | (hv[1] << 16);
                }
                const int ml = wm * 128 + i * 32 + l32;
                *reinterpret_cast<u32x2 *>(lds + ml * OUT_STRIDE + nl * 2) = u32x2{pk[0], pk[1]};
            }
        }
    __syncthreads();
    // wavefront w writes rows 32 w .. 32 w + 31, two rows per instruction;
    // 16-byte stores need every row start 16-byte aligned
    const bool vec_ok = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll 4
    for (int it = 0; it < 16; it++) {
        const int ml = wave * 32 + 2 * it + (lane >> 5);
        const int cl = (lane & 31) * 8;
        const int m = m0 + ml, n = n0 + cl;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + ml * OUT_STRIDE + cl * 2);
        if (m < M && n + 8 <= N && vec_ok) *reinterpret_cast<u32x4 *>(Y + (int64_t)m * N + n) = v;
        else if (m < M) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (n + e < N) Y[(int64_t)m * N + n + e] = (uint16_t)(v[e / 2] >> (16 * (e & 1)));
        }
    }
}


// ---------------------------------------------------------------------------
// X operand of the INT8 / FP8 decode GEMVs. Both read, for step s of
// wavefront w (k = 128 (w SPW + s) ..), the 16-byte runs 16 g and 64 + 16 g
// of X row m = min(l16, M - 1). With XS (M * SPW <= 32) each wavefront loads
// its own M x 128 SPW bytes of X once, as 16-byte chunks (chunk j = lane +
// 64 i is row j / (8 SPW), piece j % (8 SPW)), before its weight loads,
// stores them to its own LDS region and reads its fragments back after a
// wave barrier: a handful of load instructions per wavefront instead of 2 SPW
// per lane, nearly all of them repeats of the same X bytes. Otherwise each
// lane loads its fragments directly.
// Q4_GEMV_XS0 (set, not "0"): the direct X loads even where the staging
// applies (for A/B timing and the tests of both forms). Read at every call.
bool gemv_x_direct()
{
    const char *e = std::getenv("Q4_GEMV_XS0");
    return e && *e && std::strcmp(e, "0") != 0;
}

template <int SPW, bool XS>
struct GemvX {
    static constexpr int kChunks = XS ? (32 * 8 + 63) / 64 : 1;   // M * 8 SPW <= 256 chunks
    intx4 c[kChunks];
    intx4 lo[SPW], hi[SPW];

    __device__ __forceinline__ void load(const uint8_t *__restrict__ Xq, int M, int K, int s0, int m, int g,
                                         int lane)
    {
        if constexpr (XS) {
#pragma unroll
            for (int i = 0; i < kChunks; i++) {
                const int j = lane + 64 * i, r = j / (8 * SPW), p = j % (8 * SPW);
                if (r < M) c[i] = *reinterpret_cast<const intx4 *>(Xq + (int64_t)r * K + s0 * 128 + 16 * p);
            }
        } else {
#pragma unroll
            for (int s = 0; s < SPW; s++) {
                const uint8_t *xp = Xq + (int64_t)m * K + (s0 + s) * 128 + 16 * g;
                lo[s] = *reinterpret_cast<const intx4 *>(xp);
                hi[s] = *reinterpret_cast<const intx4 *>(xp + 64);
            }
        }
    }
    // xs: this wavefront's LDS region, M x 128 SPW bytes
    __device__ __forceinline__ void stage(intx4 *xs, int M, int m, int g, int lane)
    {
        if constexpr (XS) {
#pragma unroll
            for (int i = 0; i < kChunks; i++) {
                const int j = lane + 64 * i;
                if (j / (8 * SPW) < M) xs[j] = c[i];
            }
            // other lanes of this wavefront read what these lanes wrote
            asm volatile("" ::: "memory");
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int s = 0; s < SPW; s++) {
                lo[s] = xs[m * 8 * SPW + 8 * s + g];
                hi[s] = xs[m * 8 * SPW + 8 * s + 4 + g];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// FP8 decode GEMV, M <= 16, K % 1024 == 0 (K <= 8192): the E4M3 GEMM's tiles
// would use one row in 256, so a block owns 16 weight rows and its 8
// wavefronts split K into 128-k steps, each one v_mfma_scale_f32_16x16x128_
// f8f6f4 with both operands E4M3 at scale 1.0. Both operands use the same
// byte layout (a lane of group g = l / 16 holds k = 16 g .. + 15 and
// 64 + 16 g .. + 15 of the step), so weight and X fragments are loaded alike.
// Every load of a wavefront is issued at once (X first), each step is
// computed as its weight bytes land; the wavefronts' sums meet in LDS and the
// epilogue is the GEMM's, y = fp16((acc * sx[m]) * sw[n]).
constexpr int F8G_WAVES = 8;

template <int SPW, bool XS>
__global__ __launch_bounds__(F8G_WAVES * 64) void fp8_gemv16_kernel(
    const uint8_t *__restrict__ Xq, const float *__restrict__ sx, const uint8_t *__restrict__ Wq,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    __shared__ float red[F8G_WAVES][4][64];
    __shared__ intx4 xsm[XS ? F8G_WAVES * 32 * 8 : 1];   // per wavefront M x 128 SPW bytes, M * SPW <= 32
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int n0 = (int)blockIdx.x * 16;
    const int64_t nrow = n0 + l16 < N ? n0 + l16 : N - 1;
    const int m = l16 < M ? l16 : M - 1;
    const int s0 = wave * SPW;

    GemvX<SPW, XS> x;
    x.load(Xq, M, K, s0, m, g, lane);
    intx4 wlo[SPW], whi[SPW];
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        const uint8_t *wp = Wq + nrow * K + (s0 + s) * 128 + 16 * g;
        wlo[s] = *reinterpret_cast<const intx4 *>(wp);
        whi[s] = *reinterpret_cast<const intx4 *>(wp + 64);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the first product
    x.stage(xsm + wave * 32 * 8, M, m, g, lane);

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        const intx8 w8 = __builtin_shufflevector(wlo[s], whi[s], 0, 1, 2, 3, 4, 5, 6, 7);
        const intx8 a = __builtin_shufflevector(x.lo[s], x.hi[s], 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w8, a, acc, 0, 0, 0, 127, 0, 127);
    }

#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < F8G_WAVES; w++) v += red[w][r][l];
        const int mm = l & 15;                     // the result's column: X row
        const int nn = n0 + 4 * (l >> 4) + r;      // its row: weight row
        if (mm < M && nn < N) {
            float f = v * sx[mm];
            f = f * sw[nn];
            asm volatile("" : "+v"(f));   // two fp32 roundings, then fp16 (no fused multiply-convert)
            Y[(int64_t)mm * N + nn] = f2h(f);
        }
    }
}


// ---------------------------------------------------------------------------
// INT8 decode GEMV, M <= 16, K % 1024 == 0 (K <= 8192): a block owns 16 weight
// rows and its 8 wavefronts split K into 128-k steps of two
// v_mfma_i32_16x16x64_i8 each; weight and X fragments use the same byte
// layout, so they are loaded alike and the int32 sums are exact whatever the
// order. Every load is issued at once; the wavefronts' int32 partial sums meet
// in LDS; the epilogue is the GEMM's, y = fp16((float(acc) * sx[m]) * sw[n]),
// and acc_out (when given) receives the int32 sums.
constexpr int I8G_WAVES = 8;

template <int SPW, bool XS>
__global__ __launch_bounds__(I8G_WAVES * 64) void w8a8_gemv16_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    __shared__ int red[I8G_WAVES][4][64];
    __shared__ intx4 xsm[XS ? I8G_WAVES * 32 * 8 : 1];   // per wavefront M x 128 SPW bytes, M * SPW <= 32
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int n0 = (int)blockIdx.x * 16;
    const int64_t nrow = n0 + l16 < N ? n0 + l16 : N - 1;
    const int m = l16 < M ? l16 : M - 1;
    const int s0 = wave * SPW;

    GemvX<SPW, XS> x;
    x.load(reinterpret_cast<const uint8_t *>(Xq), M, K, s0, m, g, lane);
    intx4 wlo[SPW], whi[SPW];
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        const int8_t *wp = Wq + nrow * K + (s0 + s) * 128 + 16 * g;
        wlo[s] = *reinterpret_cast<const intx4 *>(wp);
        whi[s] = *reinterpret_cast<const intx4 *>(wp + 64);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the first product
    x.stage(xsm + wave * 32 * 8, M, m, g, lane);

    intx4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[s], x.lo[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[s], x.hi[s], acc, 0, 0, 0);
    }

#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
        int v = 0;
#pragma unroll
        for (int w = 0; w < I8G_WAVES; w++) v += red[w][r][l];
        const int mm = l & 15;                     // the result's column: X row
        const int nn = n0 + 4 * (l >> 4) + r;      // its row: weight row
        if (mm < M && nn < N) {
            if (acc_out) acc_out[(int64_t)mm * N + nn] = v;
            float f = (float)v * sx[mm];
            f = f * sw[nn];
            asm volatile("" : "+v"(f));   // two fp32 roundings, then fp16 (no fused multiply-convert)
            Y[(int64_t)mm * N + nn] = f2h(f);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode with the activation quantizer fused in (M * K <= 16384, M <= 16,
// K % 1024 == 0, K <= 8192): the separate per-token pass is a launch of its
// own for a few KB of X, so every block quantizes X itself. A block issues
// its X loads (one 8-element chunk per thread and pass, row-major, with the
// smoothing factors), then its weight loads, then forms x' = x / s, the
// per-row maxima (LDS max on the float bit patterns, which order as the
// values for x' >= 0), the scales max / 127 (or / 448) by IEEE division and
// the codes rint(x' / scale) -- the arithmetic of the row quantizer, so the
// codes and scales are bit for bit those of q8_quantize_act /
// fp8_quantize_act -- into LDS, while its weight bytes are on the way. The
// decode GEMV then reads its X fragments from LDS. Block 0 also writes the
// codes and scales to the caller's workspace, which therefore holds what the
// two-launch form leaves there.
template <bool FP8, bool HAS_S, int SPW>
__global__ __launch_bounds__(512) void w8a8_gemv16_fused_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ s, const uint8_t *__restrict__ Wq,
    const float *__restrict__ sw, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out, uint8_t *__restrict__ ws_codes, float *__restrict__ ws_scale)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    __shared__ __attribute__((aligned(16))) uint8_t xq[kFusedMaxMK];
    __shared__ uint32_t rmax[16];
    __shared__ float rscale[16];
    __shared__ int red[8][4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int n0 = (int)blockIdx.x * 16;
    const int64_t nrow = n0 + l16 < N ? n0 + l16 : N - 1;
    const int m = l16 < M ? l16 : M - 1;
    const int s0 = wave * SPW;
    const int nchunks = (M * K) >> 3;

    FusedX fx;
    fused_load_x<HAS_S>(fx, X, s, nchunks, K);
    intx4 wlo[SPW], whi[SPW];
#pragma unroll
    for (int t = 0; t < SPW; t++) {
        const uint8_t *wp = Wq + nrow * K + (s0 + t) * 128 + 16 * g;
        wlo[t] = *reinterpret_cast<const intx4 *>(wp);
        whi[t] = *reinterpret_cast<const intx4 *>(wp + 64);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the quantizer's arithmetic
    fused_quantize_x<FP8, HAS_S>(fx, nchunks, M, K, xq, rmax, rscale, ws_codes, ws_scale);

    // 4. the decode GEMV with its X fragments from LDS
    intx4 xlo[SPW], xhi[SPW];
#pragma unroll
    for (int t = 0; t < SPW; t++) {
        const uint8_t *xp = xq + m * K + (s0 + t) * 128 + 16 * g;
        xlo[t] = *reinterpret_cast<const intx4 *>(xp);
        xhi[t] = *reinterpret_cast<const intx4 *>(xp + 64);
    }
    if constexpr (FP8) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < SPW; t++) {
            const intx8 w8 = __builtin_shufflevector(wlo[t], whi[t], 0, 1, 2, 3, 4, 5, 6, 7);
            const intx8 a8 = __builtin_shufflevector(xlo[t], xhi[t], 0, 1, 2, 3, 4, 5, 6, 7);
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w8, a8, acc, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float pr = acc[r];   // through a scalar: bit_cast of a vector element reads element 0
            red[wave][r][lane] = __builtin_bit_cast(int, pr);
        }
    } else {
        intx4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < SPW; t++) {
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[t], xlo[t], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[t], xhi[t], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; r++) red[wave][r][lane] = acc[r];
    }
    __syncthreads();
    if (tid < 256) {
        const int r = tid >> 6, l = tid & 63;
        const int mm = l & 15;                     // the result's column: X row
        const int nn = n0 + 4 * (l >> 4) + r;      // its row: weight row
        float f;
        int vi = 0;
        if constexpr (FP8) {
            float vf = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; w++) vf += __builtin_bit_cast(float, red[w][r][l]);
            f = vf;
        } else {
#pragma unroll
            for (int w = 0; w < 8; w++) vi += red[w][r][l];
            f = (float)vi;
        }
        if (mm < M && nn < N) {
            if (!FP8 && acc_out) acc_out[(int64_t)mm * N + nn] = vi;
            f = f * rscale[mm];
            f = f * sw[nn];
            asm volatile("" : "+v"(f));   // two fp32 roundings, then fp16 (no fused multiply-convert)
            Y[(int64_t)mm * N + nn] = f2h(f);
        }
    }
}

}  // namespace

hipError_t launch_linear8_fused(const uint16_t *X, const float *s, int64_t M, int64_t N, int64_t K,
                                const uint8_t *Wq, const float *sw, uint16_t *Y, int32_t *acc_out,
                                uint8_t *ws_codes, float *ws_scale, bool fp8, hipStream_t st)
{
    if (M < 1 || M > 16 || M * K > kFusedMaxMK || K % 1024 != 0 || K > 8192 ||
        N * K >= (int64_t)1 << 31 || N < 1)
        return hipErrorNotSupported;
    const int blocks = (int)((N + 15) / 16);
    auto go = [&](auto kernel) {
        kernel<<<blocks, 512, 0, st>>>(X, s, Wq, sw, (int)M, (int)N, (int)K, Y, acc_out, ws_codes, ws_scale);
    };
#define Q4_FUSED_K(F8, HS)                                                                          \
    do {                                                                                            \
        switch (K / 1024) {                                                                         \
        case 1: go(w8a8_gemv16_fused_kernel<F8, HS, 1>); break;                                     \
        case 2: go(w8a8_gemv16_fused_kernel<F8, HS, 2>); break;                                     \
        case 4: go(w8a8_gemv16_fused_kernel<F8, HS, 4>); break;                                     \
        case 8: go(w8a8_gemv16_fused_kernel<F8, HS, 8>); break;                                     \
        default: return hipErrorNotSupported;                                                       \
        }                                                                                           \
    } while (0)
    if (fp8) { if (s) Q4_FUSED_K(true, true); else Q4_FUSED_K(true, false); }
    else { if (s) Q4_FUSED_K(false, true); else Q4_FUSED_K(false, false); }
#undef Q4_FUSED_K
    return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                            int64_t M, int64_t N, int64_t K, uint16_t *Y, int32_t *acc_out,
                            hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (M <= 16 && K % 1024 == 0 && K <= 8192 && N * K < (int64_t)1 << 31) {
        const int blocks = (int)((N + 15) / 16);
        auto go = [&](auto kernel) {
            kernel<<<blocks, I8G_WAVES * 64, 0, st>>>(Xq, sx, Wq, sw, (int)M, (int)N, (int)K, Y, acc_out);
        };
        const bool xs = M * (K / 1024) <= 32 && !gemv_x_direct();   // X staged per wavefront
        switch (K / 1024) {
        case 1: xs ? go(w8a8_gemv16_kernel<1, true>) : go(w8a8_gemv16_kernel<1, false>); return hipGetLastError();
        case 2: xs ? go(w8a8_gemv16_kernel<2, true>) : go(w8a8_gemv16_kernel<2, false>); return hipGetLastError();
        case 4: xs ? go(w8a8_gemv16_kernel<4, true>) : go(w8a8_gemv16_kernel<4, false>); return hipGetLastError();
        case 8: xs ? go(w8a8_gemv16_kernel<8, true>) : go(w8a8_gemv16_kernel<8, false>); return hipGetLastError();
        default: break;   // K = 3, 5, 6, 7 x 1024: the GEMMs
        }
    }
    if (K % (2 * LBK) == 0 && M * K < (int64_t)1 << 31 && N * K < (int64_t)1 << 31) {
        const int tiles_m = (int)((M + LBM - 1) / LBM), tiles_n = (int)((N + LBN - 1) / LBN);
        w8a8_gemm_large_kernel<false><<<tiles_m * tiles_n, 512, 0, st>>>(Xq, sx, Wq, sw, (int)M, (int)N,
                                                                        (int)K, tiles_m, Y, acc_out);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((N + QBN - 1) / QBN), (unsigned)((M + QBM - 1) / QBM));
    w8a8_gemm_kernel<<<grid, kThreads, 0, st>>>(Xq, sx, Wq, sw, (int)M, (int)N, (int)K, Y, acc_out);
    return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t *Xq, const float *sx, const uint8_t *Wq, const float *sw,
                           int64_t M, int64_t N, int64_t K, uint16_t *Y, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (K % (2 * LBK) != 0 || M * K >= (int64_t)1 << 31 || N * K >= (int64_t)1 << 31)
        return hipErrorNotSupported;
    if (M <= 16 && K % 1024 == 0 && K <= 8192) {
        const int blocks = (int)((N + 15) / 16);
        auto go = [&](auto kernel) {
            kernel<<<blocks, F8G_WAVES * 64, 0, st>>>(Xq, sx, Wq, sw, (int)M, (int)N, (int)K, Y);
        };
        const bool xs = M * (K / 1024) <= 32 && !gemv_x_direct();   // X staged per wavefront
        switch (K / 1024) {
        case 1: xs ? go(fp8_gemv16_kernel<1, true>) : go(fp8_gemv16_kernel<1, false>); return hipGetLastError();
        case 2: xs ? go(fp8_gemv16_kernel<2, true>) : go(fp8_gemv16_kernel<2, false>); return hipGetLastError();
        case 4: xs ? go(fp8_gemv16_kernel<4, true>) : go(fp8_gemv16_kernel<4, false>); return hipGetLastError();
        case 8: xs ? go(fp8_gemv16_kernel<8, true>) : go(fp8_gemv16_kernel<8, false>); return hipGetLastError();
        default: break;   // K = 3, 5, 6, 7 x 1024: the GEMM
        }
    }
    const int tiles_m = (int)((M + LBM - 1) / LBM), tiles_n = (int)((N + LBN - 1) / LBN);
    w8a8_gemm_large_kernel<true><<<tiles_m * tiles_n, 512, 0, st>>>(
        reinterpret_cast<const int8_t *>(Xq), sx, reinterpret_cast<const int8_t *>(Wq), sw, (int)M,
        (int)N, (int)K, tiles_m, Y, nullptr);
    return hipGetLastError();
}

}  // namespace q4k
