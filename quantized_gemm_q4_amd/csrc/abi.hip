// C ABI of the library (declared in include/q4.h): argument validation on the
// host, then one or two kernel launches on the caller's stream. Nothing here
// allocates; errors are reported as q4_status plus a thread-local message.
#include <cstdarg>
#include <cstdio>

#include "../../include/q4.h"
#include "q4_internal.hpp"

namespace {

constexpr int kLayoutVersion = 1;
static_assert(Q4_MAX_MULTI_LAYERS == q4k::kMaxGemvLayers, "one layer table size");
thread_local char g_err[512] = "";

q4_status fail(q4_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

q4_status ok()
{
    g_err[0] = '\0';
    return Q4_OK;
}

q4_status from_hip(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(Q4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kIntMax = 0x7fffffff;

}  // namespace

#define Q4_REQUIRE(cond, st, ...)                 \
    do {                                          \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

extern "C" {

Q4_API int q4_layout_version(void) { return kLayoutVersion; }

Q4_API const char *q4_last_error(void) { return g_err; }

Q4_API q4_status q4_quantize_pack(const void *W, int64_t N, int64_t K, int32_t g, int32_t sym,
                                  uint8_t *codes, void *scales, uint8_t *zeros, void *stream)
{
    Q4_REQUIRE(N >= 0 && K > 0 && N <= kIntMax && K <= kIntMax, Q4_ERR_INVALID_ARG,
               "q4_quantize_pack: bad shape N=%lld K=%lld", (long long)N, (long long)K);
    Q4_REQUIRE(g == 32 || g == 64 || g == 128, Q4_ERR_INVALID_ARG,
               "q4_quantize_pack: group size %d not in {32, 64, 128}", g);
    Q4_REQUIRE(K % g == 0, Q4_ERR_INVALID_ARG, "q4_quantize_pack: K=%lld not a multiple of g=%d",
               (long long)K, g);
    Q4_REQUIRE(sym == 0 || sym == 1, Q4_ERR_INVALID_ARG, "q4_quantize_pack: sym must be 0 or 1");
    if (N == 0) return ok();
    Q4_REQUIRE(W && codes && scales, Q4_ERR_INVALID_ARG, "q4_quantize_pack: null pointer");
    Q4_REQUIRE(sym || zeros, Q4_ERR_INVALID_ARG,
               "q4_quantize_pack: zeros must not be NULL when sym == 0");
    Q4_REQUIRE(aligned16(W) && aligned16(codes), Q4_ERR_MISALIGNED,
               "q4_quantize_pack: W and codes must be 16-byte aligned");
    hipError_t e = q4k::launch_q4_quantize_pack(
        static_cast<const uint16_t *>(W), N, K, g, sym, codes, static_cast<uint16_t *>(scales),
        sym ? nullptr : zeros, static_cast<hipStream_t>(stream));
    return from_hip(e, "q4_quantize_pack");
}

Q4_API q4_status w4a16_linear(const void *X, int64_t M, int64_t N, int64_t K, int32_t g,
                              const uint8_t *codes, const void *scales, const uint8_t *zeros,
                              void *Y, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= kIntMax,
               Q4_ERR_INVALID_ARG, "w4a16_linear: bad shape M=%lld N=%lld K=%lld", (long long)M,
               (long long)N, (long long)K);
    Q4_REQUIRE(g > 0 && K % g == 0 && K % 2 == 0, Q4_ERR_INVALID_ARG,
               "w4a16_linear: K=%lld must be even and a multiple of g=%d", (long long)K, g);
    Q4_REQUIRE(g % 128 == 0, Q4_ERR_UNSUPPORTED,
               "w4a16_linear: group size %d unsupported (must be a multiple of 128)", g);
    Q4_REQUIRE(M <= 65535LL * 128, Q4_ERR_UNSUPPORTED, "w4a16_linear: M=%lld too large",
               (long long)M);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && codes && scales && Y, Q4_ERR_INVALID_ARG, "w4a16_linear: null pointer");
    Q4_REQUIRE(aligned16(X) && aligned16(codes), Q4_ERR_MISALIGNED,
               "w4a16_linear: X and codes must be 16-byte aligned");
    hipError_t e = q4k::launch_w4a16(static_cast<const uint16_t *>(X), M, N, K, g, codes,
                                     static_cast<const uint16_t *>(scales), zeros,
                                     static_cast<uint16_t *>(Y), static_cast<hipStream_t>(stream));
    return from_hip(e, "w4a16_linear");
}

Q4_API q4_status w4a16_linear_multi(const void *X, int64_t M, int64_t K, int32_t g,
                                    const q4_w4a16_layer *layers, int32_t count, void *stream)
{
    Q4_REQUIRE(count >= 0 && count <= Q4_MAX_MULTI_LAYERS, Q4_ERR_INVALID_ARG,
               "w4a16_linear_multi: count=%d not in 0..%d", count, Q4_MAX_MULTI_LAYERS);
    Q4_REQUIRE(count == 0 || layers, Q4_ERR_INVALID_ARG, "w4a16_linear_multi: layers is NULL");
    Q4_REQUIRE(M >= 0 && K > 0 && M <= kIntMax && K <= kIntMax, Q4_ERR_INVALID_ARG,
               "w4a16_linear_multi: bad shape M=%lld K=%lld", (long long)M, (long long)K);
    Q4_REQUIRE(g > 0 && K % g == 0 && K % 2 == 0, Q4_ERR_INVALID_ARG,
               "w4a16_linear_multi: K=%lld must be even and a multiple of g=%d", (long long)K, g);
    Q4_REQUIRE(g % 128 == 0, Q4_ERR_UNSUPPORTED,
               "w4a16_linear_multi: group size %d unsupported (must be a multiple of 128)", g);
    Q4_REQUIRE(M <= 65535LL * 128, Q4_ERR_UNSUPPORTED, "w4a16_linear_multi: M=%lld too large",
               (long long)M);
    for (int i = 0; i < count; i++) {
        const q4_w4a16_layer &l = layers[i];
        Q4_REQUIRE(l.N >= 0 && l.N <= kIntMax, Q4_ERR_INVALID_ARG,
                   "w4a16_linear_multi: layer %d: bad N=%lld", i, (long long)l.N);
        if (M == 0 || l.N == 0) continue;
        Q4_REQUIRE(X && l.codes && l.scales && l.Y, Q4_ERR_INVALID_ARG,
                   "w4a16_linear_multi: layer %d: null pointer", i);
        Q4_REQUIRE(aligned16(X) && aligned16(l.codes), Q4_ERR_MISALIGNED,
                   "w4a16_linear_multi: layer %d: X and codes must be 16-byte aligned", i);
    }
    if (M == 0 || count == 0) return ok();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    q4k::GemvLayerDesc d[Q4_MAX_MULTI_LAYERS];
    int nd = 0;
    for (int i = 0; i < count; i++)
        if (layers[i].N > 0)
            d[nd++] = q4k::GemvLayerDesc{layers[i].codes, static_cast<const uint16_t *>(layers[i].scales),
                                         layers[i].zeros, static_cast<uint16_t *>(layers[i].Y), layers[i].N};
    if (nd == 0) return ok();
    hipError_t e = q4k::launch_w4a16_gemv_multi(static_cast<const uint16_t *>(X), M, K, g, d, nd, st);
    if (e == hipErrorNotSupported) {   // one launch per layer
        e = hipSuccess;
        for (int i = 0; i < nd && e == hipSuccess; i++)
            e = q4k::launch_w4a16(static_cast<const uint16_t *>(X), M, d[i].N, K, g, d[i].codes,
                                  d[i].scales, d[i].zeros, d[i].Y, st);
    }
    return from_hip(e, "w4a16_linear_multi");
}

static q4_status awq_scale(const char *what, const void *A, const float *awq_s, int64_t rows,
                           int64_t K, void *out, bool div, void *stream)
{
    Q4_REQUIRE(rows >= 0 && K > 0 && rows <= kIntMax && K <= kIntMax && K % 8 == 0,
               Q4_ERR_INVALID_ARG, "%s: bad shape rows=%lld K=%lld (K a multiple of 8)", what,
               (long long)rows, (long long)K);
    if (rows == 0) return ok();
    Q4_REQUIRE(A && awq_s && out, Q4_ERR_INVALID_ARG, "%s: null pointer", what);
    Q4_REQUIRE(aligned16(A) && aligned16(awq_s) && aligned16(out), Q4_ERR_MISALIGNED,
               "%s: the operands and awq_s must be 16-byte aligned", what);
    const char *a = static_cast<const char *>(A), *o = static_cast<const char *>(out);
    const size_t bytes = (size_t)rows * (size_t)K * 2;
    Q4_REQUIRE(o == a || o + bytes <= a || a + bytes <= o, Q4_ERR_INVALID_ARG,
               "%s: the output overlaps the input without being the same array", what);
    hipError_t e = q4k::launch_awq_scale(static_cast<const uint16_t *>(A), awq_s, rows, K, div,
                                         static_cast<uint16_t *>(out), static_cast<hipStream_t>(stream));
    return from_hip(e, what);
}

Q4_API q4_status awq_scale_weight(const void *W, const float *awq_s, int64_t N, int64_t K, void *Ws,
                                  void *stream)
{
    return awq_scale("awq_scale_weight", W, awq_s, N, K, Ws, false, stream);
}

Q4_API q4_status awq_scale_act(const void *X, const float *awq_s, int64_t M, int64_t K, void *Xs,
                               void *stream)
{
    return awq_scale("awq_scale_act", X, awq_s, M, K, Xs, true, stream);
}

Q4_API size_t w4a16_awq_workspace_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0) return 0;
    return ((size_t)M * (size_t)K * 2 + 255) / 256 * 256;
}

Q4_API q4_status w4a16_linear_awq(const void *X, int64_t M, int64_t N, int64_t K, int32_t g,
                                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                                  const float *awq_s, void *Y, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= kIntMax,
               Q4_ERR_INVALID_ARG, "w4a16_linear_awq: bad shape M=%lld N=%lld K=%lld", (long long)M,
               (long long)N, (long long)K);
    Q4_REQUIRE(g > 0 && K % g == 0 && K % 2 == 0, Q4_ERR_INVALID_ARG,
               "w4a16_linear_awq: K=%lld must be even and a multiple of g=%d", (long long)K, g);
    Q4_REQUIRE(g % 128 == 0, Q4_ERR_UNSUPPORTED,
               "w4a16_linear_awq: group size %d unsupported (must be a multiple of 128)", g);
    Q4_REQUIRE(M <= 65535LL * 128, Q4_ERR_UNSUPPORTED, "w4a16_linear_awq: M=%lld too large",
               (long long)M);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && codes && scales && awq_s && Y && workspace, Q4_ERR_INVALID_ARG,
               "w4a16_linear_awq: null pointer");
    Q4_REQUIRE(workspace_bytes >= w4a16_awq_workspace_bytes(M, K), Q4_ERR_INVALID_ARG,
               "w4a16_linear_awq: workspace of %zu bytes is smaller than the %zu needed",
               workspace_bytes, w4a16_awq_workspace_bytes(M, K));
    Q4_REQUIRE(aligned16(X) && aligned16(codes) && aligned16(awq_s) && aligned16(workspace),
               Q4_ERR_MISALIGNED, "w4a16_linear_awq: X, codes, awq_s and workspace must be 16-byte aligned");
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = q4k::launch_w4a16_gemv_awq(static_cast<const uint16_t *>(X), M, N, K, g, codes,
                                              static_cast<const uint16_t *>(scales), zeros, awq_s,
                                              static_cast<uint16_t *>(Y), st);
    if (e != hipErrorNotSupported) return from_hip(e, "w4a16_linear_awq");
    // other shapes: x'' into the workspace, then the plain W4A16 product
    uint16_t *xs = static_cast<uint16_t *>(workspace);
    e = q4k::launch_awq_scale(static_cast<const uint16_t *>(X), awq_s, M, K, true, xs, st);
    if (e != hipSuccess) return from_hip(e, "w4a16_linear_awq");
    e = q4k::launch_w4a16(xs, M, N, K, g, codes, static_cast<const uint16_t *>(scales), zeros,
                          static_cast<uint16_t *>(Y), st);
    return from_hip(e, "w4a16_linear_awq");
}

Q4_API q4_status q8_quantize_weight(const void *W, const float *smooth_s, int64_t N, int64_t K,
                                    int8_t *Wq, float *w_scale, void *stream)
{
    Q4_REQUIRE(N >= 0 && K > 0 && N <= kIntMax && K <= kIntMax && K % 8 == 0, Q4_ERR_INVALID_ARG,
               "q8_quantize_weight: bad shape N=%lld K=%lld (K must be a positive multiple of 8)",
               (long long)N, (long long)K);
    if (N == 0) return ok();
    Q4_REQUIRE(W && Wq && w_scale, Q4_ERR_INVALID_ARG, "q8_quantize_weight: null pointer");
    Q4_REQUIRE(aligned16(W) && aligned16(Wq) && (!smooth_s || aligned16(smooth_s)),
               Q4_ERR_MISALIGNED, "q8_quantize_weight: W, Wq and smooth_s must be 16-byte aligned");
    hipError_t e = q4k::launch_q8_weight(static_cast<const uint16_t *>(W), smooth_s, N, K, Wq,
                                         w_scale, static_cast<hipStream_t>(stream));
    return from_hip(e, "q8_quantize_weight");
}

Q4_API q4_status q8_quantize_act(const void *X, const float *smooth_s, int64_t M, int64_t K,
                                 int8_t *Xq, float *x_scale, void *stream)
{
    Q4_REQUIRE(M >= 0 && K > 0 && M <= kIntMax && K <= kIntMax && K % 8 == 0, Q4_ERR_INVALID_ARG,
               "q8_quantize_act: bad shape M=%lld K=%lld (K must be a positive multiple of 8)",
               (long long)M, (long long)K);
    if (M == 0) return ok();
    Q4_REQUIRE(X && Xq && x_scale, Q4_ERR_INVALID_ARG, "q8_quantize_act: null pointer");
    Q4_REQUIRE(aligned16(X) && aligned16(Xq) && (!smooth_s || aligned16(smooth_s)),
               Q4_ERR_MISALIGNED, "q8_quantize_act: X, Xq and smooth_s must be 16-byte aligned");
    hipError_t e = q4k::launch_q8_act(static_cast<const uint16_t *>(X), smooth_s, M, K, Xq, x_scale,
                                      static_cast<hipStream_t>(stream));
    return from_hip(e, "q8_quantize_act");
}

Q4_API q4_status w8a8_gemm(const int8_t *Xq, const float *x_scale, const int8_t *Wq,
                           const float *w_scale, int64_t M, int64_t N, int64_t K, void *Y,
                           int32_t *acc_out, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K % 16 == 0,
               Q4_ERR_INVALID_ARG,
               "w8a8_gemm: bad shape M=%lld N=%lld K=%lld (K must be a positive multiple of 16)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K <= 133143, Q4_ERR_INVALID_ARG,
               "w8a8_gemm: K=%lld could overflow the int32 accumulator (max 133143)", (long long)K);
    Q4_REQUIRE(M <= 65535LL * 128, Q4_ERR_UNSUPPORTED, "w8a8_gemm: M=%lld too large",
               (long long)M);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(Xq && x_scale && Wq && w_scale && Y, Q4_ERR_INVALID_ARG, "w8a8_gemm: null pointer");
    Q4_REQUIRE(aligned16(Xq) && aligned16(Wq), Q4_ERR_MISALIGNED,
               "w8a8_gemm: Xq and Wq must be 16-byte aligned");
    hipError_t e = q4k::launch_w8a8_gemm(Xq, x_scale, Wq, w_scale, M, N, K,
                                         static_cast<uint16_t *>(Y), acc_out,
                                         static_cast<hipStream_t>(stream));
    return from_hip(e, "w8a8_gemm");
}

Q4_API size_t w8a8_workspace_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0) return 0;
    const size_t codes = ((size_t)M * (size_t)K + 255) / 256 * 256;
    return codes + (size_t)M * sizeof(float);
}

Q4_API q4_status w8a8_linear(const void *X, int64_t M, int64_t N, int64_t K, const int8_t *Wq,
                             const float *w_scale, const float *smooth_s, void *Y, void *workspace,
                             size_t workspace_bytes, int32_t *acc_out, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K % 16 == 0 &&
                   K <= 133143,
               Q4_ERR_INVALID_ARG,
               "w8a8_linear: bad shape M=%lld N=%lld K=%lld (K a multiple of 16, <= 133143)",
               (long long)M, (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && Wq && w_scale && Y && workspace, Q4_ERR_INVALID_ARG,
               "w8a8_linear: null pointer");
    Q4_REQUIRE(workspace_bytes >= w8a8_workspace_bytes(M, K), Q4_ERR_INVALID_ARG,
               "w8a8_linear: workspace of %zu bytes is smaller than the %zu needed",
               workspace_bytes, w8a8_workspace_bytes(M, K));
    Q4_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, Q4_ERR_MISALIGNED,
               "w8a8_linear: workspace must be 256-byte aligned");
    int8_t *xq = static_cast<int8_t *>(workspace);
    float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                          ((size_t)M * (size_t)K + 255) / 256 * 256);
    q4_status st = q8_quantize_act(X, smooth_s, M, K, xq, sx, stream);
    if (st != Q4_OK) return st;
    return w8a8_gemm(xq, sx, Wq, w_scale, M, N, K, Y, acc_out, stream);
}

Q4_API q4_status fp8_quantize_weight(const void *W, const float *smooth_s, int64_t N, int64_t K,
                                     uint8_t *Wq, float *w_scale, void *stream)
{
    Q4_REQUIRE(N >= 0 && K > 0 && N <= kIntMax && K <= kIntMax && K % 8 == 0, Q4_ERR_INVALID_ARG,
               "fp8_quantize_weight: bad shape N=%lld K=%lld (K must be a positive multiple of 8)",
               (long long)N, (long long)K);
    if (N == 0) return ok();
    Q4_REQUIRE(W && Wq && w_scale, Q4_ERR_INVALID_ARG, "fp8_quantize_weight: null pointer");
    Q4_REQUIRE(aligned16(W) && aligned16(Wq) && (!smooth_s || aligned16(smooth_s)),
               Q4_ERR_MISALIGNED, "fp8_quantize_weight: W, Wq and smooth_s must be 16-byte aligned");
    hipError_t e = q4k::launch_fp8_weight(static_cast<const uint16_t *>(W), smooth_s, N, K, Wq,
                                          w_scale, static_cast<hipStream_t>(stream));
    return from_hip(e, "fp8_quantize_weight");
}

Q4_API q4_status fp8_quantize_act(const void *X, const float *smooth_s, int64_t M, int64_t K,
                                  uint8_t *Xq, float *x_scale, void *stream)
{
    Q4_REQUIRE(M >= 0 && K > 0 && M <= kIntMax && K <= kIntMax && K % 8 == 0, Q4_ERR_INVALID_ARG,
               "fp8_quantize_act: bad shape M=%lld K=%lld (K must be a positive multiple of 8)",
               (long long)M, (long long)K);
    if (M == 0) return ok();
    Q4_REQUIRE(X && Xq && x_scale, Q4_ERR_INVALID_ARG, "fp8_quantize_act: null pointer");
    Q4_REQUIRE(aligned16(X) && aligned16(Xq) && (!smooth_s || aligned16(smooth_s)),
               Q4_ERR_MISALIGNED, "fp8_quantize_act: X, Xq and smooth_s must be 16-byte aligned");
    hipError_t e = q4k::launch_fp8_act(static_cast<const uint16_t *>(X), smooth_s, M, K, Xq, x_scale,
                                       static_cast<hipStream_t>(stream));
    return from_hip(e, "fp8_quantize_act");
}

Q4_API q4_status fp8_gemm(const uint8_t *Xq, const float *x_scale, const uint8_t *Wq,
                          const float *w_scale, int64_t M, int64_t N, int64_t K, void *Y,
                          void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= 8192,
               Q4_ERR_INVALID_ARG, "fp8_gemm: bad shape M=%lld N=%lld K=%lld (K <= 8192)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K % 128 == 0, Q4_ERR_UNSUPPORTED, "fp8_gemm: K=%lld must be a multiple of 128",
               (long long)K);
    Q4_REQUIRE(M * K < (1LL << 31) && N * K < (1LL << 31), Q4_ERR_UNSUPPORTED,
               "fp8_gemm: M*K and N*K must stay below 2^31 (M=%lld N=%lld K=%lld)", (long long)M,
               (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(Xq && x_scale && Wq && w_scale && Y, Q4_ERR_INVALID_ARG, "fp8_gemm: null pointer");
    Q4_REQUIRE(aligned16(Xq) && aligned16(Wq), Q4_ERR_MISALIGNED,
               "fp8_gemm: Xq and Wq must be 16-byte aligned");
    hipError_t e = q4k::launch_fp8_gemm(Xq, x_scale, Wq, w_scale, M, N, K,
                                        static_cast<uint16_t *>(Y), static_cast<hipStream_t>(stream));
    return from_hip(e, "fp8_gemm");
}

Q4_API q4_status fp8_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *Wq,
                            const float *w_scale, const float *smooth_s, void *Y, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= 8192,
               Q4_ERR_INVALID_ARG, "fp8_linear: bad shape M=%lld N=%lld K=%lld (K <= 8192)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K % 128 == 0, Q4_ERR_UNSUPPORTED, "fp8_linear: K=%lld must be a multiple of 128",
               (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && Wq && w_scale && Y && workspace, Q4_ERR_INVALID_ARG, "fp8_linear: null pointer");
    Q4_REQUIRE(workspace_bytes >= w8a8_workspace_bytes(M, K), Q4_ERR_INVALID_ARG,
               "fp8_linear: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
               w8a8_workspace_bytes(M, K));
    Q4_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, Q4_ERR_MISALIGNED,
               "fp8_linear: workspace must be 256-byte aligned");
    uint8_t *xq = static_cast<uint8_t *>(workspace);
    float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                          ((size_t)M * (size_t)K + 255) / 256 * 256);
    q4_status st = fp8_quantize_act(X, smooth_s, M, K, xq, sx, stream);
    if (st != Q4_OK) return st;
    return fp8_gemm(xq, sx, Wq, w_scale, M, N, K, Y, stream);
}

Q4_API q4_status mxfp4_quantize_weight(const void *W, const float *smooth_s, int64_t N, int64_t K,
                                       uint8_t *codes, uint8_t *scales, void *stream)
{
    Q4_REQUIRE(N >= 0 && K > 0 && N <= kIntMax && K <= kIntMax && K % 32 == 0, Q4_ERR_INVALID_ARG,
               "mxfp4_quantize_weight: bad shape N=%lld K=%lld (K must be a positive multiple of 32)",
               (long long)N, (long long)K);
    if (N == 0) return ok();
    Q4_REQUIRE(W && codes && scales, Q4_ERR_INVALID_ARG, "mxfp4_quantize_weight: null pointer");
    Q4_REQUIRE(aligned16(W) && (!smooth_s || aligned16(smooth_s)) &&
                   (reinterpret_cast<uintptr_t>(codes) & 3u) == 0,
               Q4_ERR_MISALIGNED,
               "mxfp4_quantize_weight: W and smooth_s must be 16-byte aligned, codes 4-byte aligned");
    hipError_t e = q4k::launch_mxfp4_quantize(static_cast<const uint16_t *>(W), smooth_s, N, K, codes,
                                              scales, static_cast<hipStream_t>(stream));
    return from_hip(e, "mxfp4_quantize_weight");
}

Q4_API q4_status mxfp4_gemm(const uint8_t *Xq, const float *x_scale, const uint8_t *codes,
                            const uint8_t *scales, int64_t M, int64_t N, int64_t K, void *Y,
                            void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= 8192,
               Q4_ERR_INVALID_ARG, "mxfp4_gemm: bad shape M=%lld N=%lld K=%lld (K <= 8192)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K % 128 == 0, Q4_ERR_UNSUPPORTED, "mxfp4_gemm: K=%lld must be a multiple of 128",
               (long long)K);
    Q4_REQUIRE(M * K < (1LL << 31) && N * K < (1LL << 31), Q4_ERR_UNSUPPORTED,
               "mxfp4_gemm: M*K and N*K must stay below 2^31 (M=%lld N=%lld K=%lld)", (long long)M,
               (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(Xq && x_scale && codes && scales && Y, Q4_ERR_INVALID_ARG, "mxfp4_gemm: null pointer");
    Q4_REQUIRE(aligned16(Xq) && aligned16(codes), Q4_ERR_MISALIGNED,
               "mxfp4_gemm: Xq and codes must be 16-byte aligned");
    hipError_t e = q4k::launch_mxfp4_gemm(Xq, x_scale, codes, scales, M, N, K,
                                          static_cast<uint16_t *>(Y), static_cast<hipStream_t>(stream));
    return from_hip(e, "mxfp4_gemm");
}

Q4_API q4_status mxfp4_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                              const uint8_t *scales, const float *smooth_s, void *Y, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K <= 8192,
               Q4_ERR_INVALID_ARG, "mxfp4_linear: bad shape M=%lld N=%lld K=%lld (K <= 8192)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K % 128 == 0, Q4_ERR_UNSUPPORTED, "mxfp4_linear: K=%lld must be a multiple of 128",
               (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && codes && scales && Y && workspace, Q4_ERR_INVALID_ARG,
               "mxfp4_linear: null pointer");
    Q4_REQUIRE(workspace_bytes >= w8a8_workspace_bytes(M, K), Q4_ERR_INVALID_ARG,
               "mxfp4_linear: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
               w8a8_workspace_bytes(M, K));
    Q4_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, Q4_ERR_MISALIGNED,
               "mxfp4_linear: workspace must be 256-byte aligned");
    uint8_t *xq = static_cast<uint8_t *>(workspace);
    float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                          ((size_t)M * (size_t)K + 255) / 256 * 256);
    q4_status st = fp8_quantize_act(X, smooth_s, M, K, xq, sx, stream);
    if (st != Q4_OK) return st;
    return mxfp4_gemm(xq, sx, codes, scales, M, N, K, Y, stream);
}

Q4_API void nf4_levels(uint16_t *out)
{
    if (!out) return;
    for (int i = 0; i < 16; i++) out[i] = q4k::kNf4Levels[i];
}

Q4_API q4_status nf4_quantize(const void *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                              void *stream)
{
    Q4_REQUIRE(N >= 0 && K > 0 && N <= kIntMax && K <= kIntMax && K % 64 == 0, Q4_ERR_INVALID_ARG,
               "nf4_quantize: bad shape N=%lld K=%lld (K must be a positive multiple of 64)",
               (long long)N, (long long)K);
    if (N == 0) return ok();
    Q4_REQUIRE(W && codes && scales, Q4_ERR_INVALID_ARG, "nf4_quantize: null pointer");
    Q4_REQUIRE(aligned16(W) && (reinterpret_cast<uintptr_t>(codes) & 3u) == 0, Q4_ERR_MISALIGNED,
               "nf4_quantize: W must be 16-byte aligned, codes 4-byte aligned");
    hipError_t e = q4k::launch_nf4_quantize(static_cast<const uint16_t *>(W), N, K, codes, scales,
                                            static_cast<hipStream_t>(stream));
    return from_hip(e, "nf4_quantize");
}

Q4_API q4_status nf4_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                            const float *scales, void *Y, void *stream)
{
    Q4_REQUIRE(M >= 0 && N >= 0 && K > 0 && M <= kIntMax && N <= kIntMax && K % 128 == 0,
               Q4_ERR_INVALID_ARG, "nf4_linear: bad shape M=%lld N=%lld K=%lld (K a multiple of 128)",
               (long long)M, (long long)N, (long long)K);
    Q4_REQUIRE(K <= 28672, Q4_ERR_UNSUPPORTED, "nf4_linear: K=%lld larger than 28672", (long long)K);
    Q4_REQUIRE(N * (K / 2) < 0xFFFFFF00LL, Q4_ERR_UNSUPPORTED, "nf4_linear: weight of %lld x %lld too large",
               (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    Q4_REQUIRE(X && codes && scales && Y, Q4_ERR_INVALID_ARG, "nf4_linear: null pointer");
    Q4_REQUIRE(aligned16(X) && aligned16(codes) && (reinterpret_cast<uintptr_t>(scales) & 7u) == 0,
               Q4_ERR_MISALIGNED, "nf4_linear: X and codes must be 16-byte aligned, scales 8-byte aligned");
    hipError_t e = q4k::launch_nf4_linear(static_cast<const uint16_t *>(X), M, N, K, codes, scales,
                                          static_cast<uint16_t *>(Y), static_cast<hipStream_t>(stream));
    return from_hip(e, "nf4_linear");
}

Q4_API q4_status smoothquant_scales(const void *Xcal, int64_t R, const void *W, int64_t N,
                                    int64_t K, float alpha, float *s, void *stream)
{
    Q4_REQUIRE(R >= 1 && N >= 1 && K > 0 && K % 8 == 0, Q4_ERR_INVALID_ARG,
               "smoothquant_scales: bad shape R=%lld N=%lld K=%lld (K a multiple of 8)",
               (long long)R, (long long)N, (long long)K);
    Q4_REQUIRE(alpha >= 0.0f && alpha <= 1.0f, Q4_ERR_INVALID_ARG,
               "smoothquant_scales: alpha=%g outside [0, 1]", (double)alpha);
    Q4_REQUIRE(Xcal && W && s, Q4_ERR_INVALID_ARG, "smoothquant_scales: null pointer");
    Q4_REQUIRE(aligned16(Xcal) && aligned16(W), Q4_ERR_MISALIGNED,
               "smoothquant_scales: Xcal and W must be 16-byte aligned");
    hipError_t e = q4k::launch_smooth_scales(static_cast<const uint16_t *>(Xcal), R,
                                             static_cast<const uint16_t *>(W), N, K, alpha, s,
                                             static_cast<hipStream_t>(stream));
    return from_hip(e, "smoothquant_scales");
}

}  // extern "C"
