// AWQ-style per-input-channel scaling on the W4A16 path (Quantization
// operators guide, blog.freezetheflame.cc, §3.2: W'' = W * s and x'' = x / s
// for every input channel k; Schemes notes, lib.uml.com.cn, AWQ section:
// Y = X W = (X / s)(W * s)). Both operands stay fp16, so each scaled value is
// the IEEE fp32 product or quotient rounded once more to fp16. The search for
// s is offline; the decode GEMV fuses the activation division into its X
// staging (w4a16_gemv.hip), other shapes run this pass first.
#include "q4_internal.hpp"

namespace q4k {
namespace {

// Thread (x, y) of the grid owns the 8-column chunk blockIdx.x * 256 +
// threadIdx.x and the rows blockIdx.y, + gridDim.y, ...: its 8 factors s[k]
// are loaded once and serve every row it visits. out may be A itself (each
// element is read and written by the same thread), so neither is restrict.
template <bool DIV>
__global__ __launch_bounds__(256) void awq_scale_kernel(const uint16_t *A, const float *__restrict__ s,
                                                        int64_t rows, int64_t K, uint16_t *out)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c * 8 >= K) return;
    const floatx4 s0 = *reinterpret_cast<const floatx4 *>(s + c * 8);
    const floatx4 s1 = *reinterpret_cast<const floatx4 *>(s + c * 8 + 4);
    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(A + r * K + c * 8);
        u32x4 o;
        if constexpr (DIV) {
            o = awq_div8(v, s0, s1);
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t d = v[j];
                float lo = h2f((uint16_t)(d & 0xffffu)) * sv[2 * j];
                float hi = h2f((uint16_t)(d >> 16)) * sv[2 * j + 1];
                // keep the rounded fp32 products: without this the backend
                // folds multiply and fp16 convert into one mixed-precision
                // instruction that rounds only once
                asm volatile("" : "+v"(lo), "+v"(hi));
                o[j] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
            }
        }
        *reinterpret_cast<u32x4 *>(out + r * K + c * 8) = o;
    }
}

}  // namespace

hipError_t launch_awq_scale(const uint16_t *A, const float *s, int64_t rows, int64_t K, bool div,
                            uint16_t *out, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    const int64_t chunks = K / 8;
    const unsigned gx = (unsigned)((chunks + 255) / 256);
    // enough row slices to give the chip a few thousand blocks
    int64_t gy = (4096 + gx - 1) / gx;
    if (gy > rows) gy = rows;
    if (gy > 65535) gy = 65535;
    const dim3 grid(gx, (unsigned)gy);
    if (div) awq_scale_kernel<true><<<grid, 256, 0, st>>>(A, s, rows, K, out);
    else awq_scale_kernel<false><<<grid, 256, 0, st>>>(A, s, rows, K, out);
    return hipGetLastError();
}

}  // namespace q4k
