// Internal declarations of the gfx950 kernels' launchers and the device
// helpers they share. Not part of the ABI (see include/q4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace q4k {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt with vmcnt = n, lgkmcnt = 0, expcnt not waited (gfx9 encoding:
// vmcnt low bits 3:0 and high bits 15:14, expcnt 6:4, lgkmcnt 11:8).
#define Q4_WAIT_VM_LGKM0(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (0 << 8))

// binary16 bits <-> fp32 with the hardware converts (v_cvt_f32_f16 is exact;
// v_cvt_f16_f32 rounds to nearest even, subnormals kept).
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// AWQ-style activation scaling of eight fp16 values: f2h(h2f(x_j) / s_j),
// an IEEE fp32 division (the library is built with correctly rounded fp32
// division) rounded once more to fp16. s0 holds s_0..s_3, s1 s_4..s_7.
__device__ __forceinline__ u32x4 awq_div8(u32x4 x, floatx4 s0, floatx4 s1)
{
    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t d = x[j];
        float lo = h2f((uint16_t)(d & 0xffffu)) / sv[2 * j];
        float hi = h2f((uint16_t)(d >> 16)) / sv[2 * j + 1];
        asm volatile("" : "+v"(lo), "+v"(hi));   // the fp32 quotients, then fp16
        r[j] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
    }
    return r;
}

// Launchers. Arguments were validated by the C-ABI layer; every launcher
// enqueues on `st` and returns the launch status.
hipError_t launch_q4_quantize_pack(const uint16_t *W, int64_t N, int64_t K, int g, int sym,
                                   uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                                   hipStream_t st);
hipError_t launch_q8_weight(const uint16_t *W, const float *s, int64_t N, int64_t K,
                            int8_t *Wq, float *sw, hipStream_t st);
hipError_t launch_q8_act(const uint16_t *X, const float *s, int64_t M, int64_t K,
                         int8_t *Xq, float *sx, hipStream_t st);
// LayerNorm + SmoothQuant divide + per-token INT8 (K a multiple of 8 up to
// kLnMaxK, where the kernel's fp64 row sums are exact).
constexpr int kLnMaxK = 8192;
hipError_t launch_layernorm_quant(const uint16_t *X, const float *gamma, const float *beta, const float *s,
                                  double eps, int64_t M, int64_t K, void *Xq, float *sx, bool fp8,
                                  hipStream_t stream);
hipError_t launch_smooth_scales(const uint16_t *Xcal, int64_t R, const uint16_t *W, int64_t N,
                                int64_t K, float alpha, float *s, hipStream_t st);
hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                        const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        uint16_t *Y, hipStream_t st);
// Decode GEMV (M <= 16, g = 32, 64 or 128); hipErrorNotSupported when the shape or the
// alignment of scales / zeros does not suit it.
hipError_t launch_w4a16_gemv(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                             const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                             uint16_t *Y, hipStream_t st);

// Several decode GEMVs that read the same X (M <= 16, g = 128) in one launch,
// up to kMaxGemvLayers layers, all symmetric or all asymmetric;
// hipErrorNotSupported when the shapes or alignments do not suit it.
constexpr int kMaxGemvLayers = 8;
struct GemvLayerDesc {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint8_t *zeros;
    uint16_t *Y;
    int64_t N;
};
hipError_t launch_w4a16_gemv_multi(const uint16_t *X, int64_t M, int64_t K, int g,
                                   const GemvLayerDesc *layers, int count, hipStream_t st);
// AWQ-style per-input-channel scaling (K % 8 == 0): out = f2h(A * s[k])
// when div is false (weights), f2h(A / s[k]) when it is true (activations).
hipError_t launch_awq_scale(const uint16_t *A, const float *s, int64_t rows, int64_t K, bool div,
                            uint16_t *out, hipStream_t st);
// The decode GEMV on x'' = f2h(x / awq_s) with the division fused into its X
// staging (M == 1, g = 128); hipErrorNotSupported when it does not apply.
hipError_t launch_w4a16_gemv_awq(const uint16_t *X, int64_t M, int64_t N, int64_t K, int g,
                                 const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                                 const float *awq_s, uint16_t *Y, hipStream_t st);
hipError_t launch_w8a8_gemm(const int8_t *Xq, const float *sx, const int8_t *Wq,
                            const float *sw, int64_t M, int64_t N, int64_t K, uint16_t *Y,
                            int32_t *acc_out, hipStream_t st);
// The W8A8 (fp8 = false) or E4M3 (fp8 = true) decode layer with the per-token
// quantizer fused in: codes and scales bit for bit those of the row
// quantizer, also written to ws_codes [M, K] / ws_scale [M] by one block.
// hipErrorNotSupported unless M <= 16, M * K <= 16384, K % 1024 == 0 and
// K <= 8192; acc_out (INT8 only) as for launch_w8a8_gemm.
hipError_t launch_linear8_fused(const uint16_t *X, const float *s, int64_t M, int64_t N, int64_t K,
                                const uint8_t *Wq, const float *sw, uint16_t *Y, int32_t *acc_out,
                                uint8_t *ws_codes, float *ws_scale, bool fp8, hipStream_t st);
// FP8 E4M3 path: per-row quantizers (codes as bytes) and the GEMM (K % 128
// == 0; hipErrorNotSupported otherwise).
hipError_t launch_fp8_weight(const uint16_t *W, const float *s, int64_t N, int64_t K, uint8_t *Wq,
                             float *sw, hipStream_t st);
hipError_t launch_fp8_act(const uint16_t *X, const float *s, int64_t M, int64_t K, uint8_t *Xq,
                          float *sx, hipStream_t st);
hipError_t launch_fp8_gemm(const uint8_t *Xq, const float *sx, const uint8_t *Wq, const float *sw,
                           int64_t M, int64_t N, int64_t K, uint16_t *Y, hipStream_t st);
// MXFP4 weights (E2M1 codes [N, K/2], E8M0 block scales [N, K/32]) and the
// W4A8 GEMM with per-token E4M3 activations (K % 128 == 0 for the GEMM).
hipError_t launch_mxfp4_quantize(const uint16_t *W, const float *s, int64_t N, int64_t K,
                                 uint8_t *codes, uint8_t *scales, hipStream_t st);
hipError_t launch_mxfp4_gemm(const uint8_t *Xq, const float *sx, const uint8_t *codes,
                             const uint8_t *scales, int64_t M, int64_t N, int64_t K, uint16_t *Y,
                             hipStream_t st);
// The MXFP4 decode layer with the per-token E4M3 quantizer fused in (as
// launch_linear8_fused; also needs 16-byte aligned scales).
hipError_t launch_mxfp4_linear_fused(const uint16_t *X, const float *s, int64_t M, int64_t N, int64_t K,
                                     const uint8_t *codes, const uint8_t *scales, uint16_t *Y,
                                     uint8_t *ws_codes, float *ws_scale, hipStream_t st);
// NF4 weights (the level table is kNf4Levels in nf4_lut.hpp): the quantizer
// (codes [N, K/2], fp32 scales [N, K/64]) and the decode GEMV over row chunks
// of X (K % 128 == 0; hipErrorNotSupported otherwise).
hipError_t launch_nf4_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                               hipStream_t st);
// The NF4 form of the large-M W4A16 GEMM (tiles of 256 rows, levels times
// scales dequantized into LDS; K % 128 == 0); hipErrorNotSupported otherwise.
hipError_t launch_nf4_gemm(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                          const float *scales, uint16_t *Y, hipStream_t st);
hipError_t launch_nf4_linear(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                             const float *scales, uint16_t *Y, hipStream_t st);
// NVFP4 weights: the quantizer (codes [N, K/2], E4M3 scale bytes [N, K/16];
// K % 16 == 0), the large-M GEMM form and the layer (decode GEMV up to 48
// rows; K % 128 == 0, hipErrorNotSupported otherwise).
hipError_t launch_nvfp4_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scales,
                                 hipStream_t st);
hipError_t launch_nvfp4_gemm(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                            const uint8_t *scales, uint16_t *Y, hipStream_t st);
hipError_t launch_nvfp4_linear(const uint16_t *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                               const uint8_t *scales, uint16_t *Y, hipStream_t st);

}  // namespace q4k
