/*
 * q4.h -- C ABI of the MI355X (gfx950) group-quantized linear layer library.
 *
 * The library computes the quantized linear layer Y = X * W_hat^T of the
 * quantization pages in two forms:
 *   - W4A16: INT4 weights with one fp16 scale and one 4-bit zero-point per
 *     group of g input channels, dequantized inside the GEMM, fp16
 *     activations, fp32 accumulation, fp16 output;
 *   - W8A8: SmoothQuant-migrated per-output-channel INT8 weights, per-token
 *     dynamic INT8 activations, int32 accumulation, fp16 output;
 * and the variants the pages describe beside them: AWQ-style per-input-
 * channel scaling on the W4A16 path, FP8 E4M3 in place of INT8, MXFP4
 * weights with E4M3 activations, and NF4 weights.
 * Pages cited below:
 *   "Core ideas"        ai-infra.cypggs.com, "2. Core ideas: numeric
 *                       representation, rounding, scaling and difficulty
 *                       migration";
 *   "Operators guide"   blog.freezetheflame.cc, "Quantization operators from
 *                       basics to practice: INT8/INT4/FP8";
 *   "Method boundaries" llm-glossary.tokens-kit.com, "Method boundaries of
 *                       GPTQ, AWQ, SmoothQuant and FP8";
 *   "Quantization notes" learn.longtimenohack.com, chasing/quantization;
 *   "Schemes notes"     lib.uml.com.cn, FDE e-book, quantization-schemes.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or keeps caller memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream). Results are ready when the stream is.
 *   - fp16 means IEEE binary16 (passed as void*); all arrays are row-major
 *     and densely packed.
 *   - Arguments are checked on the host before any launch. On an error
 *     nothing is launched and nothing is written; the call returns a status
 *     and q4_last_error() holds a message (thread-local). A failed launch
 *     returns Q4_ERR_HIP. A fault inside a kernel surfaces at the caller's
 *     next synchronization. No C++ exception crosses the ABI.
 *   - A zero-sized M or N is a valid no-op.
 *   - Debug mode: with the environment variable Q4_DEBUG set (and not "0")
 *     when the library loads, every call waits for its stream after its
 *     launches, so a fault inside one of its kernels is returned by that
 *     call as Q4_ERR_HIP with the call's name in q4_last_error(), and each
 *     call writes one line ("[q4] <call>: ok" or the error) to stderr.
 *     Calls are then synchronous; off by default.
 *   - Non-finite inputs are flagged, not hidden: every quantizer gives a
 *     group (INT4 group, INT8 / E4M3 row, MXFP4 block of 32, NF4 block of
 *     64, NVFP4 block of 16) whose values -- after the smoothing multiply or
 *     divide where there is one -- hold a NaN or an infinity the format's NaN
 *     as its scale (fp16 0x7e00, fp32 0x7fc00000, E8M0 0xff, E4M3 0x7f) and
 *     0 as every code and zero-point; other groups are quantized as if it
 *     were not there. The layers then carry NaN into exactly the outputs
 *     that use a flagged group (a weight group: its output column; an
 *     activation row: its output row). Non-finite values in X of the W4A16,
 *     NF4 and NVFP4 layers, in awq_s or in smoothquant_scales' inputs give
 *     unspecified outputs (never an out-of-bounds access).
 *   - Rounding is IEEE round-to-nearest-even everywhere; divisions are true
 *     IEEE divisions. Codes, scales, zero-points and int32 accumulators are
 *     bit-reproducible.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_API __attribute__((visibility("default")))

typedef enum {
    Q4_OK = 0,
    Q4_ERR_INVALID_ARG = 1,   /* a null pointer, a bad size or shape */
    Q4_ERR_UNSUPPORTED = 2,   /* a valid request the library does not serve */
    Q4_ERR_MISALIGNED = 3,    /* a tensor pointer not 16-byte aligned */
    Q4_ERR_HIP = 4            /* the HIP runtime reported an error */
} q4_status;

/* Version of the packed layouts below (codes, scales, zeros). Bumped on any
 * change, so a stored checkpoint can be checked against the runtime's
 * packing (Method boundaries, production acceptance: the checkpoint schema
 * must match the runtime's packing). */
Q4_API int q4_layout_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
Q4_API const char *q4_last_error(void);

/* ----------------------------------------------------------------------------
 * q4_quantize_pack -- group-wise round-to-nearest INT4 quantization + packing.
 *
 * Formulas (Core ideas §2.2; Operators guide §2.1, §2.2 per-group, §3.3;
 * Quantization notes item (1) group quantization, item (2) sym/asym):
 *   asymmetric: lo = min(0, min x), hi = max(0, max x) over the group,
 *               s = fp16((hi - lo) / 15), zp = clip(rne(-lo / s), 0, 15),
 *               u = clip(rne(x / s) + zp, 0, 15);
 *   symmetric:  s = fp16(max|x| / 7), q = clip(rne(x / s), -8, 7), u = q + 8.
 * All in fp32 with true division; s is rounded once to fp16 (RNE) and the
 * codes are made from that stored scale; a scale that rounds to 0 becomes
 * 1.0. The dequantized weight is w_hat = (u - zp) * s (symmetric: zp = 8).
 *
 * W       fp16 [N, K], input, 16-byte aligned.
 * N       rows (output channels), >= 0.     K  input channels, > 0.
 * g       group size along K: 32, 64 or 128; K % g == 0.
 * sym     0 = asymmetric (zeros written), 1 = symmetric (zeros ignored).
 * codes   u8 [N, K/2] output: byte i of row n = u[n][2i] | u[n][2i+1] << 4
 *         (even k in the low nibble). 16-byte aligned.
 * scales  fp16 [N, K/g] output.
 * zeros   u8 [N, ceil(K/g/2)] output when sym == 0 (zp of group 2i in the
 *         low nibble, 2i+1 in the high nibble, 0 pads an odd count); may be
 *         NULL when sym == 1.
 * Errors: INVALID_ARG (null pointer, K % g != 0, bad g, zeros NULL with
 *         sym == 0), MISALIGNED (W or codes), HIP.
 * Storage: 4 + 16/g bits per weight symmetric, + 4/g asymmetric (4.125 and
 * 4.15625 at g = 128; Operators guide §3.3).
 * -------------------------------------------------------------------------- */
Q4_API q4_status q4_quantize_pack(const void *W, int64_t N, int64_t K, int32_t g,
                                  int32_t sym, uint8_t *codes, void *scales,
                                  uint8_t *zeros, void *stream);

/* ----------------------------------------------------------------------------
 * w4a16_linear -- Y = X * W_hat^T with the INT4 weight dequantized inside the
 * GEMM (Operators guide §1.2, the quantize/compute/dequantize pipeline fused
 * into one kernel; Method boundaries, GPTQ section: small-batch decode is
 * bound by the weight read, prefill by the dequant + matrix-core path).
 *   W_hat[n][k] = (u - zp) * s for the group of k; fp32 accumulation;
 *   Y rounded once to fp16 (RNE).
 * Accuracy: |Y - Y_ref| <= 2^-10 * sum_k |x||w_hat| (+2^-25) elementwise and
 * relative L2 <= 5e-4 against the exact product over the dequantized weight.
 *
 * X       fp16 [M, K] input, 16-byte aligned.
 * M       tokens, >= 0.   N output channels, >= 0.   K input channels, > 0.
 * g       group size: a multiple of 32 -- every size q4_quantize_pack writes
 *         (32, 64, 128) and larger multiples of 128. 128 is the layout's
 *         design point, which the decode and batched kernels serve; other
 *         sizes take general kernels that apply each group's scale to the
 *         exact fp32 sum of its own 32-wide k steps.
 * codes, scales, zeros   as written by q4_quantize_pack; zeros == NULL means
 *         symmetric (zp = 8). codes 16-byte aligned.
 * Y       fp16 [M, N] output.
 * Errors: INVALID_ARG (null pointer, K % g != 0, K % 2 != 0),
 *         UNSUPPORTED (g % 32 != 0, M > 65535 * 128), MISALIGNED (X, codes),
 *         HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status w4a16_linear(const void *X, int64_t M, int64_t N, int64_t K,
                              int32_t g, const uint8_t *codes, const void *scales,
                              const uint8_t *zeros, void *Y, void *stream);

/* ----------------------------------------------------------------------------
 * w4a16_linear_multi -- several W4A16 layers that read the same input X
 * (for example the projections that share one normalised hidden state),
 * each computed exactly as w4a16_linear defines it:
 *   Y_i = X * W_hat_i^T,   i = 0 .. count - 1.
 * With M <= 16, g == 128 and all layers symmetric or all asymmetric, the
 * layers run as one launch, so the weight stream starts and drains once for
 * all of them; otherwise (or when a layer's scale / zero-point arrays are
 * not aligned for whole-run vector loads) each layer takes its own launch.
 * Accuracy as for w4a16_linear; the k-split of the one-launch form can
 * differ from a single-layer call's, so results may differ from separate
 * w4a16_linear calls in the last bit.
 *
 * X, M, K, g   as for w4a16_linear, shared by all layers.
 * layers  HOST array of `count` descriptors (read during the call only):
 *         codes, scales, zeros as written by q4_quantize_pack for a weight
 *         [N, K] (zeros == NULL: symmetric), Y fp16 [M, N] output, N >= 0.
 * count   0 .. Q4_MAX_MULTI_LAYERS (0 is a no-op).
 * Errors: as for w4a16_linear, per layer; INVALID_ARG for a NULL `layers`
 *         with count > 0 or count out of range. Every layer is checked
 *         before anything is launched.
 * -------------------------------------------------------------------------- */
#define Q4_MAX_MULTI_LAYERS 8
typedef struct q4_w4a16_layer {
    const uint8_t *codes;
    const void *scales;
    const uint8_t *zeros;
    void *Y;
    int64_t N;
} q4_w4a16_layer;
Q4_API q4_status w4a16_linear_multi(const void *X, int64_t M, int64_t K, int32_t g,
                                    const q4_w4a16_layer *layers, int32_t count,
                                    void *stream);

/* ----------------------------------------------------------------------------
 * AWQ-style per-input-channel scaling on the W4A16 path (Operators guide
 * §3.2: W'' = W * s and x'' = x / s for every input channel k, so that
 * X W^T = (X / s)(W s)^T; Schemes notes, AWQ section). The search for s is
 * offline (outside this library); s is given, fp32 [K], finite and nonzero.
 * Both operands stay fp16: each scaled value is the IEEE fp32 product or
 * quotient rounded once more to fp16 (RNE), bit-exact with that definition.
 *
 * awq_scale_weight -- Ws[n][k] = f2h(h2f(W[n][k]) * awq_s[k]); quantize Ws
 *         with q4_quantize_pack to get the AWQ layer's packed weight.
 * awq_scale_act -- Xs[m][k] = f2h(h2f(X[m][k]) / awq_s[k]).
 * W / X fp16 [rows, K], K % 8 == 0; Ws / Xs fp16 [rows, K] output, which may
 * be the input array itself but must not partly overlap it; all three
 * pointers 16-byte aligned.
 * Errors: INVALID_ARG (shape, null pointer, partial overlap), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status awq_scale_weight(const void *W, const float *awq_s, int64_t N, int64_t K,
                                  void *Ws, void *stream);
Q4_API q4_status awq_scale_act(const void *X, const float *awq_s, int64_t M, int64_t K,
                               void *Xs, void *stream);

/* Bytes of workspace w4a16_linear_awq needs for M tokens of width K: the
 * scaled input [M, K] fp16, rounded up to 256 bytes. */
Q4_API size_t w4a16_awq_workspace_bytes(int64_t M, int64_t K);

/* ----------------------------------------------------------------------------
 * w4a16_linear_awq -- the AWQ layer at run time: Y = X'' * W_hat^T with
 * X'' = awq_scale_act(X, awq_s) and W_hat the dequantized INT4 weight of
 * awq_scale_weight(W, awq_s) (codes, scales, zeros from q4_quantize_pack).
 * With one token (M == 1, g == 128) the division is fused into the decode
 * GEMV's loads of X and the workspace is not touched; otherwise X'' is
 * written to the workspace first and w4a16_linear runs on it.
 * Accuracy as for w4a16_linear, against the exact product over X'' and
 * W_hat.
 *
 * X, M, N, K, g, codes, scales, zeros, Y   as for w4a16_linear.
 * awq_s     fp32 [K], 16-byte aligned.
 * workspace device memory of at least w4a16_awq_workspace_bytes(M, K)
 *           bytes, 16-byte aligned (required for every M).
 * Errors: as for w4a16_linear, plus INVALID_ARG for a NULL awq_s or
 *         workspace or a too small workspace, MISALIGNED for awq_s or the
 *         workspace.
 * -------------------------------------------------------------------------- */
Q4_API q4_status w4a16_linear_awq(const void *X, int64_t M, int64_t N, int64_t K, int32_t g,
                                  const uint8_t *codes, const void *scales,
                                  const uint8_t *zeros, const float *awq_s, void *Y,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------------
 * q8_quantize_weight -- per-output-channel INT8 of the smoothed weight
 * (Operators guide §2.2 per-channel, §5.1/§5.3: W' = W diag(s) folded offline;
 * Core ideas §2.4):
 *   w' = x * s[k] (fp32 multiply; smooth_s == NULL means s = 1),
 *   w_scale[n] = max(max_k |w'|, 1e-8) / 127,
 *   Wq = clip(rne(w' / w_scale[n]), -127, 127).
 * W fp16 [N, K] (16-byte aligned); smooth_s fp32 [K] or NULL;
 * Wq int8 [N, K] output (16-byte aligned); w_scale fp32 [N] output.
 * Errors: INVALID_ARG, MISALIGNED (W, Wq; K % 8 != 0 is INVALID_ARG), HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status q8_quantize_weight(const void *W, const float *smooth_s, int64_t N,
                                    int64_t K, int8_t *Wq, float *w_scale, void *stream);

/* ----------------------------------------------------------------------------
 * q8_quantize_act -- per-token dynamic INT8 of the smoothed activation
 * (Schemes notes, per-token scales computed at inference; Operators guide
 * §5.1 X / s, §5.3 the online divide):
 *   x' = x / s[k] (fp32 division; smooth_s == NULL means x' = x),
 *   x_scale[m] = max(max_k |x'|, 1e-8) / 127,
 *   Xq = clip(rne(x' / x_scale[m]), -127, 127).
 * X fp16 [M, K] (16-byte aligned); smooth_s fp32 [K] or NULL, entries finite
 * and nonzero (others give unspecified codes);
 * Xq int8 [M, K] output (16-byte aligned); x_scale fp32 [M] output.
 * Errors: INVALID_ARG (K % 8 != 0 included), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status q8_quantize_act(const void *X, const float *smooth_s, int64_t M,
                                 int64_t K, int8_t *Xq, float *x_scale, void *stream);

/* ----------------------------------------------------------------------------
 * layernorm_quant_smooth -- LayerNorm, the SmoothQuant divide and the
 * per-token INT8 quantizer in one pass (Operators guide §5.3, deployment
 * fusion: the online X / s folded into the LayerNorm epilogue, then INT8;
 * Method boundaries, SmoothQuant: the scale folded into the preceding norm).
 * Its output feeds w8a8_gemm directly, in place of q8_quantize_act on the
 * norm's fp16 output. Per row x of X:
 *   mean, var = the mean and biased variance of x, from exact sums of the
 *               fp16 values (fp64: mean = S1 / K, var = max(S2 / K - mean^2, 0)),
 *   r         = 1 / sqrt(var + eps) (fp64),
 *   x'[k]     = fl32(fma((x[k] - mean) * r, gamma[k] / s[k], beta[k] / s[k]))
 *               (fp64; smooth_s == NULL means s = 1),
 *   x_scale[m] = max(max_k |x'|, 1e-8) / 127,
 *   Xq        = clip(rne(x' / x_scale[m]), -127, 127).
 * A row holding a NaN or an infinity, or whose x' is not finite, gets a NaN
 * scale and zero codes.
 * X fp16 [M, K]; gamma, beta fp32 [K]; smooth_s fp32 [K] or NULL; Xq int8
 * [M, K] and x_scale fp32 [M] outputs. X, gamma, beta, smooth_s and Xq
 * 16-byte aligned; K a multiple of 8 up to 8192; eps > 0 and finite.
 * Errors: INVALID_ARG (shape, eps, null pointer), UNSUPPORTED (K > 8192),
 *         MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status layernorm_quant_smooth(const void *X, const float *gamma, const float *beta,
                                        const float *smooth_s, double eps, int64_t M, int64_t K,
                                        int8_t *Xq, float *x_scale, void *stream);

/* layernorm_quant_smooth_fp8 -- the same LayerNorm with the FP8 E4M3
 * per-token quantizer of fp8_quantize_act (Operators guide §4.2, §5.3):
 *   x_scale[m] = max(max_k |x'|, 1e-8) / 448,
 *   Xq = the nearest E4M3 value of fl32(x' / x_scale[m]) (ties to even, sign
 *        kept on zero), as bytes; feeds fp8_gemm.
 * Arguments, layout, flags and errors as layernorm_quant_smooth. */
Q4_API q4_status layernorm_quant_smooth_fp8(const void *X, const float *gamma, const float *beta,
                                            const float *smooth_s, double eps, int64_t M, int64_t K,
                                            uint8_t *Xq, float *x_scale, void *stream);

/* ----------------------------------------------------------------------------
 * w8a8_gemm -- INT8 GEMM with exact int32 accumulation and the scale
 * epilogue (Operators guide §2.3 INT8 GEMM + DequantizeOp, §5.2 path A):
 *   acc[m][n] = sum_k Xq[m][k] * Wq[n][k]   (exact; |acc| <= 127^2 K),
 *   Y[m][n]   = fp16(((float)acc * x_scale[m]) * w_scale[n]).
 * Xq int8 [M, K], Wq int8 [N, K] (both 16-byte aligned, K % 16 == 0 and
 * K <= 133143 so the int32 sum cannot overflow); x_scale fp32 [M];
 * w_scale fp32 [N]; Y fp16 [M, N] output; acc_out optional int32 [M, N]
 * output (for bit-exact checks; NULL in production).
 * With M <= 16 and K a multiple of 1024 up to 8192 a decode GEMV runs
 * instead of the tiles (the same exact sums and epilogue).
 * Errors: INVALID_ARG, UNSUPPORTED (M > 65535 * 128), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status w8a8_gemm(const int8_t *Xq, const float *x_scale, const int8_t *Wq,
                           const float *w_scale, int64_t M, int64_t N, int64_t K,
                           void *Y, int32_t *acc_out, void *stream);

/* Bytes of workspace w8a8_linear needs for M tokens of width K: the int8
 * codes [M, K] (rounded up to 256 bytes) followed by the fp32 scales [M]. */
Q4_API size_t w8a8_workspace_bytes(int64_t M, int64_t K);

/* ----------------------------------------------------------------------------
 * w8a8_linear -- the SmoothQuant W8A8 linear layer: q8_quantize_act of X
 * (with /smooth_s fused in) into the workspace, then w8a8_gemm.
 * smooth_s == NULL means X is already smoothed (the divide was folded into
 * the previous layer); passing s here AND folding it upstream would apply
 * it twice (Method boundaries, SmoothQuant: never apply s twice).
 * workspace: device memory of at least w8a8_workspace_bytes(M, K) bytes,
 * 256-byte aligned; after the call it holds Xq [M, K] then x_scale [M]
 * (at offset round_up(M*K, 256)).
 * Every precondition of both steps (w8a8_gemm's included) is checked before
 * the first launch. At decode sizes (M <= 16, M * K <= 16384, K a multiple of
 * 1024 up to 8192) the two steps are one launch: the decode GEMV quantizes X
 * itself (the same codes and scales bit for bit) and the workspace still
 * receives Xq and x_scale.
 * Errors: INVALID_ARG (shape as for w8a8_gemm, a null pointer, workspace too
 *         small), UNSUPPORTED (M > 65535 * 128), MISALIGNED (X, Wq,
 *         smooth_s; the workspace must be 256-byte aligned), HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status w8a8_linear(const void *X, int64_t M, int64_t N, int64_t K,
                             const int8_t *Wq, const float *w_scale,
                             const float *smooth_s, void *Y, void *workspace,
                             size_t workspace_bytes, int32_t *acc_out, void *stream);

/* ----------------------------------------------------------------------------
 * w8a8_linear_noalloc -- w8a8_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, the same kernels and the same
 * results bit for bit, with the per-token codes and scales kept in a scratch
 * array the library holds in device memory instead of a caller workspace.
 * The call itself allocates nothing.
 *
 * Scratch: Q4_NOALLOC_SCRATCH_BYTES (16 MiB + 64 KiB) per GPU, a fixed array
 * each GPU the library runs on holds until the process ends; its device
 * address is looked up on the first call on each device. A call needs
 * w8a8_workspace_bytes(M, K) of it (M * K rounded up to 256, plus 4 M): the
 * W8A8 workload's 2048 x 8192 fits. Larger M * K is refused with
 * UNSUPPORTED before anything runs.
 * Every call on one GPU shares that GPU's array and leaves its codes and
 * scales in it: calls that overlap on one GPU (two streams, two threads)
 * race on it and must be serialised by the caller. Nothing in it has to
 * start at zero (each call writes what it reads).
 * The stream must belong to the current device (hipSetDevice).
 *
 * X, M, N, K, Wq, w_scale, smooth_s, Y, acc_out, stream: as for w8a8_linear.
 * Errors: as for w8a8_linear (no workspace arguments), plus UNSUPPORTED for
 *         a request beyond the scratch array and HIP if the array's address
 *         cannot be found.
 * -------------------------------------------------------------------------- */
#define Q4_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u + 64u * 1024u)
Q4_API size_t w8a8_noalloc_max_bytes(void);
Q4_API q4_status w8a8_linear_noalloc(const void *X, int64_t M, int64_t N, int64_t K,
                                     const int8_t *Wq, const float *w_scale,
                                     const float *smooth_s, void *Y, int32_t *acc_out,
                                     void *stream);

/* ----------------------------------------------------------------------------
 * FP8 E4M3 variant of the W8A8 path (Operators guide §4.1 formats: E4M3 for
 * weights and activations; §4.2 scaled FP8 GEMM, C = scale_A * scale_B *
 * (A_fp8 @ B_fp8); Core ideas §2.1: E4M3 range +-448). The scales are
 * per output channel and per token as in the INT8 path, with 448 for 127.
 * Codes are OCP E4M3 bytes (bias 7, S.1111.111 is NaN and never produced).
 *
 * fp8_quantize_weight / fp8_quantize_act -- per-row E4M3 of W diag(s) /
 * of X / s (smooth_s == NULL: s = 1):
 *   v = w * s[k] (weights) or x / s[k] (activations, IEEE fp32),
 *   scale[row] = max(max_k |v|, 1e-8) / 448,
 *   q = e4m3(v / scale): the nearest E4M3 value, ties to even, sign kept on
 *       zero (the quotient never exceeds 448 by more than rounding).
 * Codes and scales are bit-exact with the IEEE definition.
 * W / X fp16 [rows, K] (16-byte aligned, K % 8 == 0); smooth_s fp32 [K] or
 * NULL (16-byte aligned); codes u8 [rows, K] (16-byte aligned); scale fp32
 * [rows]. Errors: INVALID_ARG, MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status fp8_quantize_weight(const void *W, const float *smooth_s, int64_t N,
                                     int64_t K, uint8_t *Wq, float *w_scale, void *stream);
Q4_API q4_status fp8_quantize_act(const void *X, const float *smooth_s, int64_t M,
                                  int64_t K, uint8_t *Xq, float *x_scale, void *stream);

/* ----------------------------------------------------------------------------
 * fp8_gemm -- E4M3 GEMM with fp32 accumulation and the scale epilogue:
 *   acc[m][n] = sum_k e4m3(Xq[m][k]) * e4m3(Wq[n][k])   (fp32 sums of exact
 *               products, in the matrix cores' order),
 *   Y[m][n]   = fp16((acc * x_scale[m]) * w_scale[n]).
 * Accuracy: |Y - Y_ref| <= 2^-10 * x_scale w_scale sum_k |products| (+2^-25)
 * against the exact sum (K <= 8192 keeps the fp32 sum within half of it).
 * With M <= 16 and K a multiple of 1024 a decode GEMV runs instead of the
 * 256 x 256 tiles (same formula and bound, another summation order).
 * Xq, Wq u8 E4M3 codes [M, K], [N, K] (16-byte aligned); x_scale fp32 [M];
 * w_scale fp32 [N]; Y fp16 [M, N] output. K must be a multiple of 128;
 * M*K and N*K below 2^31.
 * Errors: INVALID_ARG (shape; K > 8192), UNSUPPORTED (K % 128 != 0, M*K or
 *         N*K >= 2^31), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status fp8_gemm(const uint8_t *Xq, const float *x_scale, const uint8_t *Wq,
                          const float *w_scale, int64_t M, int64_t N, int64_t K, void *Y,
                          void *stream);

/* ----------------------------------------------------------------------------
 * fp8_linear -- fp8_quantize_act of X (with /smooth_s fused in) into the
 * workspace, then fp8_gemm; the workspace is sized and laid out as for
 * w8a8_linear (w8a8_workspace_bytes(M, K) bytes, 256-byte aligned: E4M3 codes
 * [M, K], then x_scale [M] at offset round_up(M*K, 256)). smooth_s as for
 * w8a8_linear. Every precondition of both steps is checked before the
 * first launch; at decode sizes the two steps are one launch, as for
 * w8a8_linear. Errors: as for fp8_gemm, plus a too small or misaligned
 * workspace and a misaligned X or smooth_s.
 * -------------------------------------------------------------------------- */
Q4_API q4_status fp8_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *Wq,
                            const float *w_scale, const float *smooth_s, void *Y,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------------
 * MXFP4 weights with E4M3 activations (W4A8) (Operators guide §4.3: FP4
 * E2M1 elements sharing one E8M0 scale per block of 32, weights in FP4 and
 * activations kept in FP8; Schemes notes: E2M1 = {0, +-0.5, ..., +-4, +-6}).
 *
 * mxfp4_quantize_weight -- per row n and block j of 32 along K:
 *   v = w * s[k] (fp32; smooth_s == NULL: s = 1), amax = max_block |v|,
 *   scale = 2^(e - 127), e = the smallest integer >= 1 with
 *           amax <= 6 * 2^(e - 127) (e = 0 for an all-zero block),
 *   code = e2m1(v / scale): the nearest E2M1 value, ties to the even code,
 *          sign kept on zero (|v / scale| <= 6 by the choice of e).
 * W fp16 [N, K] (16-byte aligned, K % 32 == 0); smooth_s fp32 [K] or NULL
 * (16-byte aligned); codes u8 [N, K/2] output, two codes per byte along K
 * (even k in the low nibble), 4-byte aligned; scales u8 [N, K/32] output
 * (E8M0). 4.25 bits per weight. Codes and scales are bit-exact.
 * Errors: INVALID_ARG, MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status mxfp4_quantize_weight(const void *W, const float *smooth_s, int64_t N,
                                       int64_t K, uint8_t *codes, uint8_t *scales,
                                       void *stream);

/* ----------------------------------------------------------------------------
 * mxfp4_gemm -- W4A8 GEMM on the scaled matrix cores:
 *   acc[m][n] = sum_k e4m3(Xq[m][k]) * e2m1(code[n][k]) * 2^(scales[n][k/32] - 127)
 *               (fp32 sums of exact products, in the matrix cores' order),
 *   Y[m][n]   = fp16(acc * x_scale[m]).
 * Accuracy: |Y - Y_ref| <= 2^-10 * x_scale sum_k |products| (+2^-25).
 * With M <= 32 and K a multiple of 1024 (scales 16-byte aligned) a decode
 * GEMV runs instead of the 256 x 256 tiles; the sums' order differs, the
 * accuracy bound is the same.
 * Xq u8 E4M3 [M, K] and x_scale fp32 [M] as written by fp8_quantize_act;
 * codes, scales as written by mxfp4_quantize_weight (Xq and codes 16-byte
 * aligned); Y fp16 [M, N] output. K a multiple of 128, at most 8192; M*K
 * and N*K below 2^31.
 * Errors: INVALID_ARG (shape, K > 8192), UNSUPPORTED (K % 128 != 0, M*K or
 *         N*K >= 2^31), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status mxfp4_gemm(const uint8_t *Xq, const float *x_scale, const uint8_t *codes,
                            const uint8_t *scales, int64_t M, int64_t N, int64_t K, void *Y,
                            void *stream);

/* ----------------------------------------------------------------------------
 * mxfp4_linear -- fp8_quantize_act of X (with /smooth_s fused in) into the
 * workspace (laid out as for w8a8_linear, w8a8_workspace_bytes(M, K) bytes,
 * 256-byte aligned), then mxfp4_gemm. smooth_s as for w8a8_linear.
 * Every precondition of both steps is checked before the first launch; at
 * decode sizes (as for w8a8_linear, with 16-byte aligned scales) the two
 * steps are one launch.
 * Errors: as for mxfp4_gemm, plus a too small or misaligned workspace and a
 * misaligned X or smooth_s.
 * -------------------------------------------------------------------------- */
Q4_API q4_status mxfp4_linear(const void *X, int64_t M, int64_t N, int64_t K,
                              const uint8_t *codes, const uint8_t *scales,
                              const float *smooth_s, void *Y, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------------
 * NF4 weights (Operators guide §3.4: 16 non-uniform levels, the medians of
 * 16 equal-probability intervals of N(0, 1), scaled to [-1, 1] and kept in
 * fp16; one fp32 scale, the block's max |w|, per block of 64 weights; code =
 * the index of the level nearest to w / scale; w_hat = level[code] * scale).
 *
 * nf4_levels -- copies the 16 levels (fp16 bit patterns, ascending:
 *   Phi^-1((i + 0.5) / 16) / Phi^-1(31 / 32) rounded to fp16) to the HOST
 *   array `out`. No GPU work.
 * nf4_quantize -- scale = max(max_block |w|, 1e-8); x = w / scale (IEEE
 *   fp32); code = the first index minimising fabsf(x - level[i]) in fp32.
 *   W fp16 [N, K] (16-byte aligned, K % 64 == 0); codes u8 [N, K/2] output,
 *   two codes per byte along K (even k in the low nibble), 4-byte aligned;
 *   scales fp32 [N, K/64] output. Codes and scales are bit-exact.
 * nf4_linear -- Y = X * W_hat^T, fp32 accumulation, fp16 output. Up to 48
 *   rows (decode): the levels enter the matrix cores exactly and each
 *   64-block's fp32 partial sum is multiplied by its scale; X is processed in
 *   passes of at most 16 rows (at most 8 when 9 rows of X do not fit the
 *   LDS), each pass reading the whole weight once. Above 48 rows (prefill): a
 *   tiled GEMM that reads the weight once per tile of rows, with
 *   w_hat = level * scale rounded once to fp16 as the matrix-core operand
 *   (the scale is taken as fp16, which every scale nf4_quantize writes is).
 *   X fp16 [M, K] and codes 16-byte aligned; scales 8-byte aligned;
 *   K % 128 == 0; Y fp16 [M, N] output.
 * Accuracy: as for w4a16_linear (decode: as its GEMV; above 48 rows: as its
 *   large-M GEMM, one fp16 rounding of w_hat).
 * Errors: INVALID_ARG, UNSUPPORTED (N * K / 2 >= 2^32 - 256: the weight
 *   outgrows the kernels' 32-bit offsets), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API void nf4_levels(uint16_t *out);
Q4_API q4_status nf4_quantize(const void *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                              void *stream);
Q4_API q4_status nf4_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                            const float *scales, void *Y, void *stream);

/* ----------------------------------------------------------------------------
 * NVFP4 weights (Quantization notes, FP4 item: FP4 E2M1 values with one FP8
 * E4M3 scale per block of 16 along K, 4 + 8/16 = 4.5 bits per weight; its
 * NVFP4-style sketch: scale = E4M3(amax / 6), code = the E2M1 value of
 * w / scale, clipped to +-6).
 *
 * nvfp4_quantize -- per block of 16: scale = e4m3(fl32(amax / 6)) (nearest,
 *   ties to even, saturating at 448); code = e2m1(fl32(w / scale)) (nearest,
 *   ties to even, saturating at 6, sign kept on zero), or 0 for every weight
 *   of a block whose scale is 0 (amax / 6 at most 2^-10);
 *   w_hat = e2m1(code) * e4m3(scale). W fp16 [N, K] (16-byte aligned,
 *   K % 16 == 0); codes u8 [N, K/2] output, two codes per byte along K (even
 *   k in the low nibble), 4-byte aligned; scales u8 [N, K/16] output, E4M3
 *   bytes. Codes and scales are bit-exact.
 * nvfp4_linear -- Y = X * W_hat^T, fp32 accumulation, fp16 output. w_hat is
 *   exact in fp16 (at most 6 significant bits, within [2^-10, 2688]), so the
 *   block scale is folded into the fp16 matrix-core operand without a
 *   rounding. Up to 48 rows: a decode GEMV, passes of at most 16 rows, each
 *   reading the weight once; above 48 rows the tiled GEMM of w4a16_linear.
 *   X fp16 [M, K] and codes 16-byte aligned; scales 2-byte aligned;
 *   K % 128 == 0; Y fp16 [M, N] output.
 * Accuracy: |Y - Y_ref| <= 2^-10 * sum_k |x||w_hat| (+2^-25) elementwise
 *   against the exact product over the dequantized weight.
 * Errors: INVALID_ARG, UNSUPPORTED (N * K / 2 >= 2^32 - 256), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status nvfp4_quantize(const void *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scales,
                                void *stream);
Q4_API q4_status nvfp4_linear(const void *X, int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                              const uint8_t *scales, void *Y, void *stream);

/* ----------------------------------------------------------------------------
 * smoothquant_scales -- the SmoothQuant migration factor from calibration
 * activations (Operators guide §5.1; Core ideas §2.4; Quantization notes,
 * SmoothQuant):
 *   s[j] = max(ax_j, 1e-8)^alpha / max(aw_j, 1e-8)^(1 - alpha),
 *   ax_j = max_r |Xcal[r][j]|, aw_j = max_n |W[n][j]|.
 * At alpha == 0.5 the powers are correctly rounded square roots and s is
 * bit-reproducible; other alpha in [0, 1] use powf (within a few ulp).
 * Xcal fp16 [R, K], W fp16 [N, K] (both 16-byte aligned, K % 8 == 0);
 * s fp32 [K] output. This is an offline step; it is not on the hot path.
 * Errors: INVALID_ARG (R or N < 1, alpha outside [0, 1]), MISALIGNED, HIP.
 * -------------------------------------------------------------------------- */
Q4_API q4_status smoothquant_scales(const void *Xcal, int64_t R, const void *W,
                                    int64_t N, int64_t K, float alpha, float *s,
                                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
