// MXFP4 weights with FP8 E4M3 activations (W4A8) on gfx950 (Quantization
// operators guide §4.3: FP4 E2M1 elements with one E8M0 scale per block of
// 32, weights in FP4 while the activations stay in FP8; Core ideas §2.1 and
// the Schemes notes: E2M1 holds {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}).
//
// Layout: codes [N, K/2], two E2M1 codes per byte along K (even k in the low
// nibble), scales [N, K/32] E8M0 bytes (value 2^(e - 127)). The activations
// are the per-token E4M3 codes and fp32 scales of fp8_quantize_act.
//
// The GEMM runs on v_mfma_scale_f32_32x32x64_f8f6f4 with the weight as the
// first operand (format E2M1) and X as the second (format E4M3): each weight
// lane supplies 32 consecutive k of one row, i.e. exactly one MX block, with
// that block's E8M0 byte as its scale operand; X's scale operand is 1.0 (127).
// Products are exact in fp32; the sums are fp32 in the matrix cores' order;
// the epilogue is y = fp16(acc * x_scale[m]).
#include <type_traits>

#include "fp4_codes.hpp"
#include "q4_internal.hpp"
#include "row_codes.hpp"

namespace q4k {
namespace {

// ---------------------------------------------------------------------------
// Quantizer. A lane owns 8 consecutive weights of a row (one 16-byte load),
// four lanes one block of 32; the block's max |v| is a quad reduction. The
// scale is the smallest power of two 2^(e - 127) with amax <= 6 * 2^(e - 127),
// found from amax's exponent with one exact comparison (e = 0 for an all-zero
// block); v * 2^(127 - e) is exact, and e2m1_code (fp4_codes.hpp) counts it
// against the format's rounding thresholds with ties to the even code.

// max over a quad of |v| bit patterns (NaN and the infinities rank above
// every finite value)
__device__ __forceinline__ uint32_t quad_max_bits(uint32_t a)
{
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false));   // quad swap 1 0 3 2
    return max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false));   // quad swap 2 3 0 1
}

template <bool HAS_S>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const uint16_t *__restrict__ W,
                                                             const float *__restrict__ s, int64_t N,
                                                             int64_t K, uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales)
{
    const int64_t chunks = K >> 3;                        // 8-weight chunks per row
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = c < N * chunks;
    const int64_t cc = live ? c : N * chunks - 1;         // idle lanes redo the last chunk
    const int64_t row = cc / chunks, k0 = (cc % chunks) * 8;
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(W + row * K + k0);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = h2f((uint16_t)(raw[i] & 0xffffu));
        v[2 * i + 1] = h2f((uint16_t)(raw[i] >> 16));
    }
    if (HAS_S) {
        const floatx4 a = *reinterpret_cast<const floatx4 *>(s + k0);
        const floatx4 b = *reinterpret_cast<const floatx4 *>(s + k0 + 4);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[i] *= a[i];
            v[4 + i] *= b[i];
        }
    }
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __builtin_bit_cast(uint32_t, v[i]) & 0x7fffffffu);
    const uint32_t amax_bits = quad_max_bits(m);   // the four lanes of a block are a quad (K % 32 == 0)
    // a block holding a NaN or an infinity is flagged: scale byte 0xff
    // (E8M0's NaN), codes 0
    const bool bad = amax_bits >= 0x7f800000u;
    const float amax = bad ? 0.0f : __builtin_bit_cast(float, amax_bits);
    int e = 0;
    if (amax > 0.0f) {
        int ex;
        const float f = frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
        // 6 * 2^(e - 127) = 0.75 * 2^(e - 124): e = ex + 124 if f <= 0.75, else ex + 125
        e = ex + 124 + (f > 0.75f ? 1 : 0);
        e = e < 1 ? 1 : (e > 254 ? 254 : e);
    }
    // 2^(127 - e), exact (a subnormal only at e = 254); an all-zero block
    // multiplies by 0, which keeps every code 0 and every sign
    const float mul = e == 0 ? 0.0f : ldexpf(1.0f, 127 - e);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) out |= e2m1_code(v[i] * mul) << (4 * i);
    if (live) {
        *reinterpret_cast<uint32_t *>(codes + row * (K >> 1) + (k0 >> 1)) = bad ? 0u : out;
        if ((threadIdx.x & 3) == 0) scales[row * (K >> 5) + (k0 >> 5)] = bad ? (uint8_t)0xff : (uint8_t)e;
    }
}

// ---------------------------------------------------------------------------
// W4A8 GEMM. The 256 x 256 tile kernel of the INT8 / FP8 path with a stage
// per 64 k of: X 256 rows x 64 B (E4M3), W 256 rows x 32 B (E2M1) and the
// W block scales 256 rows x 2 blocks, six stages (156 KB) filled by direct
// global-to-LDS loads five steps ahead. Per stage a wavefront issues two X
// loads (16 rows x 64 B each, 16-byte chunks XOR-swizzled by (row >> 2) & 3),
// one W load (32 rows x 32 B, the two halves of a row swapped when row bit 3
// is set: a gfx950 ds_read_b128 serves 16 lanes per cycle, four 4-lane groups
// sharing lane bit 5 and the parity of lane bits 2-4, so unswizzled rows r
// and r + 24 or r + 8 of one group met in a bank) and one byte load of 64 scale bytes (32 rows x
// 2 blocks; a byte-sized direct load still fills one dword of LDS per lane,
// so the scale of row r, block h sits at dword 2 r + h), so the wait counts
// are those of the FP8 kernel. The 8
// wavefronts form a 2 (M) x 4 (N) grid of 128 x 64 sub-tiles; each step is
// one MFMA per 32 x 32 tile (4 before the barrier, 4 after it, interleaved
// with the next stage's reads). Accumulator tiles are Y transposed (the
// weight is the first operand): a lane holds one row of Y and four
// consecutive columns per group of four registers; the epilogue stages the
// fp16 tile in LDS and writes whole rows with 16-byte stores.
//
// With K % 512 == 0 (SG = true) the scales take another route: every 8 steps
// wavefronts 0-3 load the next 8 steps' scales of the tile's 256 rows (16
// bytes per row, one 16-byte load per lane) into one of two 4 KB LDS
// buffers, so a step's scale traffic is 32 requests of 16 bytes instead of
// 256 single bytes. Those loads are issued after the step's stage loads:
// for wavefronts 0-3 the fixed wait counts then also cover them (a stricter
// wait, never a looser one), and the group is first read 7 steps later,
// after the wait for a younger stage and a barrier.
constexpr int MBM = 256, MBN = 256, MBK = 64, MSTAGES = 6;
constexpr int MW_BYTES = MBN * MBK / 2;                   // 8 KB of codes
constexpr int MOUT_STRIDE = MBN * 2 + 16;
// a stage: X (BM rows x 64 B), the codes, the per-step scales (!SG)
template <int BM> constexpr int mx_bytes = BM * MBK;
template <bool SG> constexpr int ms_bytes = SG ? 0 : MBN * 2 * 4;   // per-step scales, one per dword
template <bool SG, int BM> constexpr int mstage_bytes = mx_bytes<BM> + MW_BYTES + ms_bytes<SG>;
constexpr int MSG_BYTES = 2 * MBN * 16;                   // two groups of 8 steps' scales
template <bool SG, int BM>
constexpr int mlds_bytes = BM * MOUT_STRIDE > MSTAGES * mstage_bytes<SG, BM> + (SG ? MSG_BYTES : 0)
                               ? BM * MOUT_STRIDE
                               : MSTAGES * mstage_bytes<SG, BM> + (SG ? MSG_BYTES : 0);

// BM = 256: the whole tile. BM = 128 (a half tile, 64 x 64 per wavefront)
// serves the tiles past the last full round of 256 blocks two CUs each, so
// that, for example, the 344 tiles of a 2048 x 11008 output take one round
// of full tiles and one of half tiles instead of two rounds of full ones;
// tile0 is the first tile the launch covers.
template <bool SG, int BM = MBM>
__global__ __launch_bounds__(512, 1) void mxfp4_gemm_kernel(
    const uint8_t *__restrict__ Xq, const float *__restrict__ sx, const uint8_t *__restrict__ Wc,
    const uint8_t *__restrict__ Ws, int M, int N, int K, int tiles_m, int tile0, uint16_t *__restrict__ Y)
{
    static_assert(BM == 256 || BM == 128, "full or half tiles");
    constexpr int MT = BM / 64;                  // 32-row tiles per wavefront
    constexpr int XL = BM / 128;                 // X loads per stage and wavefront
    constexpr int MX_BYTES = mx_bytes<BM>;
    constexpr int MSTAGE_BYTES = mstage_bytes<SG, BM>;
    constexpr int LPS = XL + (SG ? 1 : 2);       // direct loads per stage and wavefront
    __shared__ __attribute__((aligned(1024))) uint8_t lds[mlds_bytes<SG, BM>];
    uint8_t *const sreg = lds + MSTAGES * MSTAGE_BYTES;   // SG: the two scale groups

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, h = lane >> 5;
    const int blocks = gridDim.x, b = blockIdx.x;
    const int ub = (blocks % 8 == 0) ? (b % 8) * (blocks / 8) + b / 8 : b;
    const int t = tile0 + (BM == MBM ? ub : ub >> 1);
    const int m0 = (t % tiles_m) * MBM + (BM == MBM ? 0 : (ub & 1) * BM), n0 = (t / tiles_m) * MBN;
    const int KT = K / MBK;
    const uint32_t KC = (uint32_t)K >> 1, KS = (uint32_t)K >> 5;   // bytes per code / scale row

    // direct-load addresses (rows past M or N read the last row)
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    // (a fixed-size array: one sized by a template parameter and captured by
    // the lambda below makes this compiler drop the kernel's host stub)
    uint32_t xoff[2];
#pragma unroll
    for (int j = 0; j < XL; j++) {
        int m = m0 + (XL * wave + j) * 16 + (lane >> 2);
        m = m < M ? m : M - 1;
        xoff[j] = (uint32_t)m * (uint32_t)K + 16 * dchunk;
    }
    int nw = n0 + wave * 32 + (lane >> 1);
    nw = nw < N ? nw : N - 1;
    // the two 16-byte halves of a code row are swapped on rows with bit 3 set
    // (row 32 wave + lane / 2: bit 3 is lane bit 4), so that the fragment
    // reads below, 32 rows of one half, are free of LDS bank conflicts
    const uint32_t woff = (uint32_t)nw * KC + 16 * ((lane & 1) ^ ((lane >> 4) & 1));
    const uint32_t soff = (uint32_t)nw * KS + (lane & 1);
    auto issue = [&](uint8_t *stage, int kt) {
#pragma unroll
        for (int j = 0; j < XL; j++)
            __builtin_amdgcn_global_load_lds(Xq + xoff[j] + (uint32_t)kt * MBK, stage + (XL * wave + j) * 1024,
                                             16, 0, 0);
        __builtin_amdgcn_global_load_lds(Wc + woff + (uint32_t)kt * 32, stage + MX_BYTES + wave * 1024, 16, 0, 0);
        if constexpr (!SG)
            __builtin_amdgcn_global_load_lds(Ws + soff + (uint32_t)kt * 2, stage + MX_BYTES + MW_BYTES + wave * 256,
                                             1, 0, 0);
    };
    // SG: scale group g (steps 8g .. 8g + 7) into buffer g & 1; wavefront w
    // < 4 loads rows 64 w .. 64 w + 63, lane i row 64 w + i (past the end:
    // the last group again)
    int ns = n0 + (wave & 3) * 64 + lane;
    ns = ns < N ? ns : N - 1;
    const uint32_t sgoff = (uint32_t)ns * KS;
    const int ngroups = KT >> 3;
    auto issue_scales = [&](int g) {
        if (SG && wave < 4) {
            const int gg = g < ngroups ? g : ngroups - 1;
            __builtin_amdgcn_global_load_lds(Ws + sgoff + (uint32_t)gg * 16, sreg + (g & 1) * 4096 + wave * 1024,
                                             16, 0, 0);
        }
    };

    // Operand layout of the instruction with these formats (measured): an
    // E2M1 lane of half h holds k = 32h .. 32h + 31 of the 64-k step, one MX
    // block, and its scale is that block's; an E4M3 lane of half h holds
    // k = 16h .. 16h + 15 in bytes 0-15 and k = 32 + 16h .. 32 + 16h + 15 in
    // bytes 16-31. So: X row wm*128 + 32 i + l32, logical chunks h and 2 + h;
    // W row wn*64 + 32 j + l32, code bytes 16h .. 16h + 15; its scale in
    // dword 2 row + h.
    const int swz = (l32 >> 2) & 3;
    const int xa = (wm * (BM / 2) + l32) * MBK, xc0 = 16 * (h ^ swz), xc1 = 16 * ((2 + h) ^ swz);
    const int wrow = wn * 64 + l32;
    const int wb = MX_BYTES + wrow * 32 + 16 * (h ^ ((l32 >> 3) & 1));   // half h of row wrow (swapped on bit 3)
    const int sb = MX_BYTES + MW_BYTES + (wrow * 2 + h) * 4;   // !SG: inside the stage
    const int sgb = wrow * 16 + h;                              // SG: inside a scale group

    floatx16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    struct Frags {
        intx8 a[MT];
        intx4 w[2];
        int s[2];
    };
    auto read = [&](const uint8_t *stage, int step, Frags &f) {
#pragma unroll
        for (int i = 0; i < MT; i++) {
            const intx4 lo = *reinterpret_cast<const intx4 *>(stage + xa + i * 32 * MBK + xc0);
            const intx4 hi = *reinterpret_cast<const intx4 *>(stage + xa + i * 32 * MBK + xc1);
            f.a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            f.w[j] = *reinterpret_cast<const intx4 *>(stage + wb + j * 32 * 32);
            if constexpr (SG) f.s[j] = sreg[((step >> 3) & 1) * 4096 + sgb + j * 32 * 16 + 2 * (step & 7)];
            else f.s[j] = stage[sb + j * 32 * 2 * 4];
        }
    };
    auto mma_half = [&](const Frags &f, int s) {   // row tiles i = s MT / 2 .. (s + 1) MT / 2 - 1
#pragma unroll
        for (int i = s * MT / 2; i < (s + 1) * MT / 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const intx8 w8 = __builtin_shufflevector(f.w[j], intx4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
                // first operand E2M1 (format 4) with its block scale, second E4M3 (format 0) at 1.0
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, f.a[i], acc[i][j], 4, 0, 0,
                                                                             f.s[j], 0, 127);
            }
    };

    // Software pipeline as in the INT8 / FP8 kernel (six stages here).
    issue_scales(0);
#pragma unroll
    for (int p = 0; p < MSTAGES; p++) issue(lds + p * MSTAGE_BYTES, p < KT ? p : KT - 1);
    Frags f[2];
    asm volatile("" ::: "memory");
    Q4_WAIT_VM_LGKM0(LPS * (MSTAGES - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read(lds, 0, f[0]);
    int sc = 0;   // stage of step k (k mod 6)
    for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int k = kt + u;
            const int sn = sc == MSTAGES - 1 ? 0 : sc + 1;
            mma_half(f[u], 0);
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            Q4_WAIT_VM_LGKM0(LPS * (MSTAGES - 2));   // loads outstanding: stages k + 2 .. k + 5
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            read(lds + sn * MSTAGE_BYTES, k + 1, f[u ^ 1]);
            issue(lds + sc * MSTAGE_BYTES, k + MSTAGES < KT ? k + MSTAGES : KT - 1);
            if (SG && (k & 7) == 0) issue_scales((k >> 3) + 1);
            mma_half(f[u], 1);
            if constexpr (BM == MBM) {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (g >= 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // VMEM read
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);               // DS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
                }
            } else {
#pragma unroll
                for (int g = 0; g < 2; g++) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);               // VMEM read
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);               // DS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
                }
            }
            sc = sn;
        }
    }
    Q4_WAIT_VM_LGKM0(0);   // the refetches past the end

    // Epilogue: y = f2h(acc * sx[m]) through an LDS-staged fp16 tile
    float xsv[MT];
#pragma unroll
    for (int i = 0; i < MT; i++) {
        const int m = m0 + wm * (BM / 2) + i * 32 + l32;
        xsv[i] = sx[m < M ? m : M - 1];
    }
    __syncthreads();   // every wavefront is done with the stages
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int nl = wn * 64 + j * 32 + 8 * q + 4 * h;
#pragma unroll
            for (int i = 0; i < MT; i++) {
                uint32_t pk[2];
#pragma unroll
                for (int e2 = 0; e2 < 2; e2++) {
                    const uint32_t lo = f2h(acc[i][j][4 * q + 2 * e2] * xsv[i]);
                    const uint32_t hi = f2h(acc[i][j][4 * q + 2 * e2 + 1] * xsv[i]);
                    pk[e2] = lo | (hi << 16);
                }
                const int ml = wm * (BM / 2) + i * 32 + l32;
                *reinterpret_cast<u32x2 *>(lds + ml * MOUT_STRIDE + nl * 2) = u32x2{pk[0], pk[1]};
            }
        }
    __syncthreads();
    const bool vec_ok = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll 4
    for (int it = 0; it < BM / 16; it++) {
        const int ml = wave * (BM / 8) + 2 * it + (lane >> 5);
        const int cl = (lane & 31) * 8;
        const int m = m0 + ml, n = n0 + cl;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + ml * MOUT_STRIDE + cl * 2);
        if (m < M && n + 8 <= N && vec_ok) *reinterpret_cast<u32x4 *>(Y + (int64_t)m * N + n) = v;
        else if (m < M) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (n + e < N) Y[(int64_t)m * N + n + e] = (uint16_t)(v[e / 2] >> (16 * (e & 1)));
        }
    }
}

// ---------------------------------------------------------------------------
// Decode GEMV, M <= 32, K % 1024 == 0 (K <= 8192): the same scaled
// instruction with 32 weight rows per block and the block's 16 wavefronts
// splitting K into SPW 64-k steps each. A wavefront issues its X fragments,
// its block scales (one vector load) and then the code runs of all its steps
// at once, so the whole packed weight is in flight from the start, and each
// step is computed as soon as its code run has landed. X rows past M repeat
// row M - 1 (the MFMA's columns do not mix and those are never stored). The
// wavefronts' partial sums meet in LDS in a fixed order; y = fp16(acc * sx[m]).

//
// With XL (M (K + 16) <= 64 KB) the block first stages X in LDS (rows K + 16
// bytes apart, so the 16-byte operand reads of 16 rows fall in distinct
// banks; one broadcast read when M = 1) and the wavefronts read their
// fragments there: one or two global loads per thread instead of two per
// step per wavefront. The stage shares its LDS with the final reduction.
constexpr int MXG_WAVES = 16;
constexpr int MXG_LDS = MXG_WAVES * 16 * 64 * 4;   // 64 KB

template <int SPW, bool XL>
__global__ __launch_bounds__(MXG_WAVES * 64) void mxfp4_gemv_kernel(
    const uint8_t *__restrict__ Xq, const float *__restrict__ sx, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int M, int N, int K, uint16_t *__restrict__ Y)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    __shared__ __attribute__((aligned(16))) unsigned char lds[MXG_LDS];
    float(*red)[16][64] = reinterpret_cast<float(*)[16][64]>(lds);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int n0 = (int)blockIdx.x * 32;
    const uint32_t nrow = (uint32_t)(n0 + l32 < N ? n0 + l32 : N - 1);
    const int m = l32 < M ? l32 : M - 1;
    const int s0 = wave * SPW;                     // first 64-k step of this wavefront
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 5;
    const int xs = K + 16;                         // LDS row stride of the staged X

    // X: row m, k = 64 s + 16 h .. + 15 (bytes 0-15) and 64 s + 32 + 16 h .. + 15
    intx4 xlo[SPW], xhi[SPW];
    constexpr int XPT = MXG_LDS / 16 / (MXG_WAVES * 64);   // 16-byte chunks per thread at most
    intx4 xv[XPT];
    const int nch = XL ? M * (K >> 4) : 0;
    if (XL) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int c = (int)threadIdx.x + i * MXG_WAVES * 64;
            if (c < nch) xv[i] = *reinterpret_cast<const intx4 *>(Xq + (size_t)c * 16);
        }
    } else {
#pragma unroll
        for (int s = 0; s < SPW; s++) {
            const uint8_t *xp = Xq + (size_t)m * (size_t)K + (size_t)(s0 + s) * 64 + 16 * h;
            xlo[s] = *reinterpret_cast<const intx4 *>(xp);
            xhi[s] = *reinterpret_cast<const intx4 *>(xp + 32);
        }
    }
    // the row's 2 SPW block scales from step s0 on (byte 2 s + h is step s's)
    uint32_t sc[(2 * SPW + 3) / 4];
    {
        const uint8_t *sp = scales + nrow * ks + 2u * (uint32_t)s0;
        if constexpr (SPW == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(sp);
#pragma unroll
            for (int e = 0; e < 4; e++) sc[e] = a[e];
        } else if constexpr (SPW == 4) {
            const u32x2 a = *reinterpret_cast<const u32x2 *>(sp);
            sc[0] = a[0];
            sc[1] = a[1];
        } else if constexpr (SPW == 2) {
            sc[0] = *reinterpret_cast<const uint32_t *>(sp);
        } else {
            sc[0] = *reinterpret_cast<const uint16_t *>(sp);
        }
    }
    intx4 cw[SPW];
#pragma unroll
    for (int s = 0; s < SPW; s++)
        cw[s] = *reinterpret_cast<const intx4 *>(codes + nrow * kh + (uint32_t)(s0 + s) * 32u + 16u * (uint32_t)h);
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the first product
    if (XL) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int c = (int)threadIdx.x + i * MXG_WAVES * 64;
            const int r = c / (K >> 4), cc = c - r * (K >> 4);
            if (c < nch) *reinterpret_cast<intx4 *>(lds + r * xs + cc * 16) = xv[i];
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SPW; s++) {
            const unsigned char *xp = lds + m * xs + (s0 + s) * 64 + 16 * h;
            xlo[s] = *reinterpret_cast<const intx4 *>(xp);
            xhi[s] = *reinterpret_cast<const intx4 *>(xp + 32);
        }
    }

    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        const intx8 w8 = __builtin_shufflevector(cw[s], intx4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
        const intx8 a = __builtin_shufflevector(xlo[s], xhi[s], 0, 1, 2, 3, 4, 5, 6, 7);
        const uint32_t word = sc[(2 * s + h) >> 2];
        const int e = (int)((word >> (8 * ((2 * s + h) & 3))) & 0xffu);
        // first operand E2M1 (format 4) with its block scale, second E4M3 (format 0) at 1.0
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, a, acc, 4, 0, 0, e, 0, 127);
    }

    if (XL) __syncthreads();   // every wavefront has read its X fragments
#pragma unroll
    for (int r = 0; r < 16; r++) red[wave][r][lane] = acc[r];
    __syncthreads();
    {
        const int r = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < MXG_WAVES; w++) v += red[w][r][l];
        const int mm = l & 31;                                  // the accumulator's column: X row
        const int nn = n0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);   // its row: weight row
        if (mm < M && nn < N) Y[(int64_t)mm * N + nn] = f2h(v * sx[mm]);
    }
}

// ---------------------------------------------------------------------------
// Decode GEMV for M <= 16 on v_mfma_scale_f32_16x16x128_f8f6f4: 16 weight
// rows per block (twice the blocks of the 32-row kernel above, so the grid
// spreads evenly over the CUs), 8 wavefronts splitting K into SPW 128-k steps
// (one instruction each). Operand layout of the instruction (measured): an
// E2M1 lane of group g = l / 16 holds k = 32 g .. 32 g + 31 of the step (its
// MX block, so its scale is that block's byte), an E4M3 lane of group g holds
// k = 16 g .. + 15 in bytes 0-15 and k = 64 + 16 g .. + 15 in bytes 16-31;
// result lane l holds X row l % 16 and weight rows 4 (l / 16) .. + 3. Loads,
// X staging (XL: M (K + 16) <= 32 KB) and the final sum as in the 32-row kernel.
constexpr int MXH_WAVES = 8;
constexpr int MXH_LDS = 32 * 1024;

template <int SPW, bool XL>
__global__ __launch_bounds__(MXH_WAVES * 64) void mxfp4_gemv16_kernel(
    const uint8_t *__restrict__ Xq, const float *__restrict__ sx, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int M, int N, int K, uint16_t *__restrict__ Y)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    __shared__ __attribute__((aligned(16))) unsigned char lds[MXH_LDS];
    float(*red)[4][64] = reinterpret_cast<float(*)[4][64]>(lds);   // [MXH_WAVES][4][64]: 8 KB
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int n0 = (int)blockIdx.x * 16;
    const uint32_t nrow = (uint32_t)(n0 + l16 < N ? n0 + l16 : N - 1);
    const int m = l16 < M ? l16 : M - 1;
    const int s0 = wave * SPW;                     // first 128-k step of this wavefront
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 5;
    const int xs = K + 16;

    intx4 xlo[SPW], xhi[SPW];
    constexpr int XPT = MXH_LDS / 16 / (MXH_WAVES * 64);
    intx4 xv[XPT];
    const int nch = XL ? M * (K >> 4) : 0;
    if (XL) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int c = (int)threadIdx.x + i * MXH_WAVES * 64;
            if (c < nch) xv[i] = *reinterpret_cast<const intx4 *>(Xq + (size_t)c * 16);
        }
    } else {
#pragma unroll
        for (int s = 0; s < SPW; s++) {
            const uint8_t *xp = Xq + (size_t)m * (size_t)K + (size_t)(s0 + s) * 128 + 16 * g;
            xlo[s] = *reinterpret_cast<const intx4 *>(xp);
            xhi[s] = *reinterpret_cast<const intx4 *>(xp + 64);
        }
    }
    // the row's 4 SPW block scales from step s0 on (byte 4 s + g is step s's)
    uint32_t sc[SPW];
    {
        const uint8_t *sp = scales + nrow * ks + 4u * (uint32_t)s0;
        if constexpr (SPW == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(sp);
            const u32x4 b = *reinterpret_cast<const u32x4 *>(sp + 16);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                sc[e] = a[e];
                sc[4 + e] = b[e];
            }
        } else if constexpr (SPW == 4) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(sp);
#pragma unroll
            for (int e = 0; e < 4; e++) sc[e] = a[e];
        } else if constexpr (SPW == 2) {
            const u32x2 a = *reinterpret_cast<const u32x2 *>(sp);
            sc[0] = a[0];
            sc[1] = a[1];
        } else {
            sc[0] = *reinterpret_cast<const uint32_t *>(sp);
        }
    }
    intx4 cw[SPW];
#pragma unroll
    for (int s = 0; s < SPW; s++)
        cw[s] = *reinterpret_cast<const intx4 *>(codes + nrow * kh + (uint32_t)(s0 + s) * 64u + 16u * (uint32_t)g);
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the first product
    if (XL) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int c = (int)threadIdx.x + i * MXH_WAVES * 64;
            const int r = c / (K >> 4), cc = c - r * (K >> 4);
            if (c < nch) *reinterpret_cast<intx4 *>(lds + r * xs + cc * 16) = xv[i];
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SPW; s++) {
            const unsigned char *xp = lds + m * xs + (s0 + s) * 128 + 16 * g;
            xlo[s] = *reinterpret_cast<const intx4 *>(xp);
            xhi[s] = *reinterpret_cast<const intx4 *>(xp + 64);
        }
    }

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPW; s++) {
        const intx8 w8 = __builtin_shufflevector(cw[s], intx4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
        const intx8 a = __builtin_shufflevector(xlo[s], xhi[s], 0, 1, 2, 3, 4, 5, 6, 7);
        const int e = (int)((sc[s] >> (8 * g)) & 0xffu);
        // first operand E2M1 (format 4) with its block scale, second E4M3 (format 0) at 1.0
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w8, a, acc, 4, 0, 0, e, 0, 127);
    }

    if (XL) __syncthreads();   // every wavefront has read its X fragments
#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < MXH_WAVES; w++) v += red[w][r][l];
        const int mm = l & 15;                     // the result's column: X row
        const int nn = n0 + 4 * (l >> 4) + r;      // its row: weight row
        if (mm < M && nn < N) Y[(int64_t)mm * N + nn] = f2h(v * sx[mm]);
    }
}

// The decode GEMV above with the per-token E4M3 quantizer of its input fused
// in (M * K <= 16384): every block quantizes X into LDS (fused_quantize_x,
// bit for bit fp8_quantize_act) while its weight bytes are in flight, then
// runs the same 16-row MFMA chain with its X fragments from LDS. Block 0
// also writes the codes and scales to the caller's workspace.
template <int SPW, bool HAS_S>
__global__ __launch_bounds__(MXH_WAVES * 64) void mxfp4_gemv16_fused_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ s, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int M, int N, int K, uint16_t *__restrict__ Y,
    uint8_t *__restrict__ ws_codes, float *__restrict__ ws_scale)
{
    static_assert(SPW == 1 || SPW == 2 || SPW == 4 || SPW == 8, "steps per wavefront");
    static_assert(MXH_WAVES * 64 == 512, "the fused quantizer takes 512 threads");
    __shared__ __attribute__((aligned(16))) uint8_t xq[kFusedMaxMK];
    __shared__ uint32_t rmax[16];
    __shared__ float rscale[16];
    __shared__ float red[MXH_WAVES][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int n0 = (int)blockIdx.x * 16;
    const uint32_t nrow = (uint32_t)(n0 + l16 < N ? n0 + l16 : N - 1);
    const int m = l16 < M ? l16 : M - 1;
    const int s0 = wave * SPW;
    const uint32_t kh = (uint32_t)K >> 1, ks = (uint32_t)K >> 5;
    const int nchunks = (M * K) >> 3;

    FusedX fx;
    fused_load_x<HAS_S>(fx, X, s, nchunks, K);
    uint32_t sc[SPW];
    {
        const uint8_t *sp = scales + nrow * ks + 4u * (uint32_t)s0;
        if constexpr (SPW == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(sp);
            const u32x4 b = *reinterpret_cast<const u32x4 *>(sp + 16);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                sc[e] = a[e];
                sc[4 + e] = b[e];
            }
        } else if constexpr (SPW == 4) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(sp);
#pragma unroll
            for (int e = 0; e < 4; e++) sc[e] = a[e];
        } else if constexpr (SPW == 2) {
            const u32x2 a = *reinterpret_cast<const u32x2 *>(sp);
            sc[0] = a[0];
            sc[1] = a[1];
        } else {
            sc[0] = *reinterpret_cast<const uint32_t *>(sp);
        }
    }
    intx4 cw[SPW];
#pragma unroll
    for (int t = 0; t < SPW; t++)
        cw[t] = *reinterpret_cast<const intx4 *>(codes + nrow * kh + (uint32_t)(s0 + t) * 64u + 16u * (uint32_t)g);
    __builtin_amdgcn_sched_barrier(0);   // every load goes out before the quantizer's arithmetic
    fused_quantize_x<true, HAS_S>(fx, nchunks, M, K, xq, rmax, rscale, ws_codes, ws_scale);

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < SPW; t++) {
        const uint8_t *xp = xq + m * K + (s0 + t) * 128 + 16 * g;
        const intx4 xlo = *reinterpret_cast<const intx4 *>(xp);
        const intx4 xhi = *reinterpret_cast<const intx4 *>(xp + 64);
        const intx8 w8 = __builtin_shufflevector(cw[t], intx4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
        const intx8 a = __builtin_shufflevector(xlo, xhi, 0, 1, 2, 3, 4, 5, 6, 7);
        const int e = (int)((sc[t] >> (8 * g)) & 0xffu);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w8, a, acc, 4, 0, 0, e, 0, 127);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int r = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < MXH_WAVES; w++) v += red[w][r][l];
        const int mm = l & 15;                     // the result's column: X row
        const int nn = n0 + 4 * (l >> 4) + r;      // its row: weight row
        if (mm < M && nn < N) Y[(int64_t)mm * N + nn] = f2h(v * rscale[mm]);
    }
}

}  // namespace

hipError_t launch_mxfp4_linear_fused(const uint16_t *X, const float *s, int64_t M, int64_t N, int64_t K,
                                     const uint8_t *codes, const uint8_t *scales, uint16_t *Y,
                                     uint8_t *ws_codes, float *ws_scale, hipStream_t st)
{
    if (M < 1 || M > 16 || M * K > kFusedMaxMK || K % 1024 != 0 || K > 8192 ||
        N * K >= (int64_t)1 << 31 || N < 1 || (reinterpret_cast<uintptr_t>(scales) & 15) != 0)
        return hipErrorNotSupported;
    const int blocks = (int)((N + 15) / 16);
    auto go = [&](auto k_s, auto k_n) {
        if (s) k_s<<<blocks, MXH_WAVES * 64, 0, st>>>(X, s, codes, scales, (int)M, (int)N, (int)K, Y, ws_codes, ws_scale);
        else k_n<<<blocks, MXH_WAVES * 64, 0, st>>>(X, s, codes, scales, (int)M, (int)N, (int)K, Y, ws_codes, ws_scale);
    };
    switch (K / 1024) {
    case 1: go(mxfp4_gemv16_fused_kernel<1, true>, mxfp4_gemv16_fused_kernel<1, false>); break;
    case 2: go(mxfp4_gemv16_fused_kernel<2, true>, mxfp4_gemv16_fused_kernel<2, false>); break;
    case 4: go(mxfp4_gemv16_fused_kernel<4, true>, mxfp4_gemv16_fused_kernel<4, false>); break;
    case 8: go(mxfp4_gemv16_fused_kernel<8, true>, mxfp4_gemv16_fused_kernel<8, false>); break;
    default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

hipError_t launch_mxfp4_quantize(const uint16_t *W, const float *s, int64_t N, int64_t K,
                                 uint8_t *codes, uint8_t *scales, hipStream_t st)
{
    if (N == 0) return hipSuccess;
    const int64_t threads = N * (K >> 3);
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (s) mxfp4_quantize_kernel<true><<<(unsigned)grid, 256, 0, st>>>(W, s, N, K, codes, scales);
    else mxfp4_quantize_kernel<false><<<(unsigned)grid, 256, 0, st>>>(W, s, N, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mxfp4_gemm(const uint8_t *Xq, const float *sx, const uint8_t *codes,
                             const uint8_t *scales, int64_t M, int64_t N, int64_t K, uint16_t *Y,
                             hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    if (K % (2 * MBK) != 0 || M * K >= (int64_t)1 << 31 || N * K >= (int64_t)1 << 31)
        return hipErrorNotSupported;
    if (M <= 16 && K % 1024 == 0 && K <= 8192 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) {
        const int blocks = (int)((N + 15) / 16);
        const bool xl = M * (K + 16) <= MXH_LDS;
        auto go = [&](auto k_lds, auto k_reg) {
            if (xl) k_lds<<<blocks, MXH_WAVES * 64, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, Y);
            else k_reg<<<blocks, MXH_WAVES * 64, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, Y);
        };
        switch (K / 1024) {
        case 1: go(mxfp4_gemv16_kernel<1, true>, mxfp4_gemv16_kernel<1, false>); break;
        case 2: go(mxfp4_gemv16_kernel<2, true>, mxfp4_gemv16_kernel<2, false>); break;
        case 4: go(mxfp4_gemv16_kernel<4, true>, mxfp4_gemv16_kernel<4, false>); break;
        case 8: go(mxfp4_gemv16_kernel<8, true>, mxfp4_gemv16_kernel<8, false>); break;
        default: goto gemm;
        }
        return hipGetLastError();
    }
    if (M <= 32 && K % 1024 == 0 && K <= 8192 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) {
        const int blocks = (int)((N + 31) / 32);
        const bool xl = M * (K + 16) <= MXG_LDS;
        auto go = [&](auto k_lds, auto k_reg) {
            if (xl) k_lds<<<blocks, MXG_WAVES * 64, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, Y);
            else k_reg<<<blocks, MXG_WAVES * 64, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, Y);
        };
        switch (K / 1024) {
        case 1: go(mxfp4_gemv_kernel<1, true>, mxfp4_gemv_kernel<1, false>); break;
        case 2: go(mxfp4_gemv_kernel<2, true>, mxfp4_gemv_kernel<2, false>); break;
        case 4: go(mxfp4_gemv_kernel<4, true>, mxfp4_gemv_kernel<4, false>); break;
        case 8: go(mxfp4_gemv_kernel<8, true>, mxfp4_gemv_kernel<8, false>); break;
        default: goto gemm;   // K = 3, 5, 6, 7, ... x 1024
        }
        return hipGetLastError();
    }
gemm:
    const int tiles_m = (int)((M + MBM - 1) / MBM), tiles_n = (int)((N + MBN - 1) / MBN);
    const int tiles = tiles_m * tiles_n;
    // whole rounds of 256 full tiles, then the rest as half tiles when they
    // fit one round of 256 blocks (and the full tiles fill at least one)
    const int full = tiles > 256 && 2 * (tiles % 256) <= 256 ? tiles - tiles % 256 : tiles;
    // 16-byte scale group loads need whole, aligned 16-byte runs per row
    const bool sg = K % 512 == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0;
    auto go = [&](auto k_full, auto k_half) {
        k_full<<<full, 512, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, tiles_m, 0, Y);
        if (full < tiles)
            k_half<<<2 * (tiles - full), 512, 0, st>>>(Xq, sx, codes, scales, (int)M, (int)N, (int)K, tiles_m,
                                                       full, Y);
    };
    if (sg) go(mxfp4_gemm_kernel<true, MBM>, mxfp4_gemm_kernel<true, MBM / 2>);
    else go(mxfp4_gemm_kernel<false, MBM>, mxfp4_gemm_kernel<false, MBM / 2>);
    return hipGetLastError();
}

}  // namespace q4k
