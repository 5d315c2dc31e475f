/*
 * oracle.c -- plain, slow CPU oracle for the group-quantized linear layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library. The product path
 * (the HIP library under quantized_gemm_q4_amd/) shares no code with it and
 * never calls it.
 *
 * Every function follows the formulas of the quantization pages, written out
 * step by step with no blocking, fusion or reordering:
 *   - "Quantization operators guide" = blog.freezetheflame.cc, "Quantization
 *     operators from basics to practice: INT8/INT4/FP8".
 *   - "Core ideas" = ai-infra.cypggs.com, "2. Core ideas: numeric
 *     representation, rounding, scaling and difficulty migration".
 *   - "Method boundaries" = llm-glossary.tokens-kit.com, "Method boundaries
 *     of GPTQ, AWQ, SmoothQuant and FP8".
 *   - "Quantization notes" = learn.longtimenohack.com, chasing/quantization.
 *
 * Arithmetic rules. The quantizers decide integers (codes, zero-points) from
 * floating point, so they run in IEEE binary32 with round-to-nearest-even:
 * true division, no FMA contraction (built with -ffp-contract=off), rintf()
 * under the default FE_TONEAREST mode. The GEMM references are exact: fp64
 * sums of exactly dequantized operands (W4A16) and int64 sums (W8A8).
 *
 * Non-finite inputs: every quantizer flags a group (or row) whose values hold
 * a NaN or an infinity with the format's NaN scale and zero codes; the GEMM
 * references carry NaN into the outputs that use such a group.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds
 * zero and the subnormals (fraction * 2^-24), exponent 31 holds Inf/NaN.
 * (Core ideas, §2.1: FP16 = 1 + 5 + 10, range +-65504.)                     */

float orc_h2f(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);                 /* subnormal or zero */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25);     /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a binary32 value to the nearest binary16, ties to even. The value is
 * written as r * q with q the binary16 spacing of its binade (2^-24 below the
 * normal range); r is rounded to the nearest integer with ties to even, which
 * is the same as an even last fraction bit. Magnitudes >= 65520 (half-way
 * between 65504 and 2^16) round to infinity.                                 */
uint16_t orc_f2h(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return sign | 0x7e00;
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                 /* a = fr * 2^ex, fr in [0.5, 1) */
    int b = ex - 1;                /* binade: 2^b <= a < 2^(b+1)     */
    double q = (b < -14) ? ldexp(1.0, -24) : ldexp(1.0, b - 10);
    double r = nearbyint(a / q);   /* a / q is exact; ties to even   */
    double v = r * q;              /* the rounded magnitude           */
    if (v == 0.0)
        return sign;
    if (v < ldexp(1.0, -14))       /* subnormal result */
        return sign | (uint16_t)(v / ldexp(1.0, -24));
    frexp(v, &ex);
    b = ex - 1;
    if (b > 15)
        return sign | 0x7c00;
    uint16_t frac = (uint16_t)(v / ldexp(1.0, b - 10) - 1024.0);
    return sign | (uint16_t)((b + 15) << 10) | frac;
}

void orc_h2f_array(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_h2f(h[i]);
}

void orc_f2h_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_f2h(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Group-wise INT4 RTN quantizer.
 *
 * Asymmetric (Core ideas §2.2; Quantization operators guide §2.1):
 *   s = (max - min) / (2^b - 1),  zp = round(-min / s),
 *   q = clip(round(x / s) + zp, 0, 2^b - 1),  x_hat = (q - zp) * s.
 * Symmetric (Core ideas §2.2):
 *   s = max|x| / (2^(b-1) - 1),  q = clip(round(x / s), -2^(b-1), 2^(b-1) - 1).
 * One fp16 scale and one zero-point per group of g consecutive elements of a
 * weight row (Quantization notes, item (1) group quantization; Quantization
 * operators guide §2.2 per-group, §3.3). Rounding is to nearest, ties to
 * even (Core ideas §2.2).
 *
 * Readings where the pages leave a step open:
 *   - the range is widened to contain 0 (lo = min(0, min x), hi = max(0,
 *     max x)), so zp stays in [0, 15] and 0 is exact; on a group with both
 *     signs this is the pages' formula unchanged;
 *   - s is computed in fp32 and rounded once to the stored fp16 scale; the
 *     codes are made from that stored scale, so quantize and dequantize use
 *     the same s; a scale that rounds to 0 is replaced by 1.0;
 *   - round first, then add zp (the order the formula is written in);
 *   - true division x / s, not a multiply by 1/s;
 *   - symmetric codes are stored offset-binary, u = q + 8;
 *   - a group holding a NaN or an infinity is flagged: its scale is the fp16
 *     NaN 0x7e00 and its codes and zero-point are 0 (the other groups are
 *     quantized as if it were not there).
 * Packing: codes[n][i] = u[n][2i] | u[n][2i+1] << 4 (even k in the low
 * nibble); zeros[n][i] = zp[n][2i] | zp[n][2i+1] << 4, a zero nibble pads an
 * odd group count. All arrays row-major.                                    */

static void quant_group(const uint16_t *w, int g, int sym, uint8_t *u,
                        uint16_t *scale16, int *zp_out)
{
    for (int k = 0; k < g; k++) {
        if (!isfinite(orc_h2f(w[k]))) {        /* flagged group: NaN scale, codes and zp 0 */
            for (int j = 0; j < g; j++) u[j] = 0;
            *scale16 = 0x7e00;
            *zp_out = 0;
            return;
        }
    }
    float lo = 0.0f, hi = 0.0f, amax = 0.0f;
    for (int k = 0; k < g; k++) {
        float x = orc_h2f(w[k]);
        if (x < lo) lo = x;
        if (x > hi) hi = x;
        if (fabsf(x) > amax) amax = fabsf(x);
    }
    float s32 = sym ? amax / 7.0f : (hi - lo) / 15.0f;
    uint16_t s16 = orc_f2h(s32);
    if ((s16 & 0x7fff) == 0)
        s16 = 0x3c00;                          /* 1.0 */
    float sf = orc_h2f(s16);
    int zp;
    if (sym) {
        zp = 8;
    } else {
        float z = rintf(-lo / sf);
        zp = (int)z;
        if (zp < 0) zp = 0;
        if (zp > 15) zp = 15;
    }
    for (int k = 0; k < g; k++) {
        float x = orc_h2f(w[k]);
        int q = (int)rintf(x / sf);
        if (sym) {
            if (q < -8) q = -8;
            if (q > 7) q = 7;
            u[k] = (uint8_t)(q + 8);
        } else {
            q += zp;
            if (q < 0) q = 0;
            if (q > 15) q = 15;
            u[k] = (uint8_t)q;
        }
    }
    *scale16 = s16;
    *zp_out = zp;
}

/* W fp16 [N, K] -> codes u8 [N, K/2], scales fp16 [N, K/g],
 * zeros u8 [N, ceil(K/g/2)] (asymmetric only; ignored when sym).
 * Returns 0, or -1 on a shape it does not accept.                           */
int orc_q4_quantize_pack(const uint16_t *W, int64_t N, int64_t K, int g,
                         int sym, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros)
{
    if (N < 0 || K <= 0 || g <= 0 || K % g != 0 || K % 2 != 0 || g % 2 != 0)
        return -1;
    int64_t G = K / g, Gz = (G + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        uint8_t *u = (uint8_t *)malloc((size_t)K);
        int *zp = (int *)malloc(sizeof(int) * (size_t)G);
        for (int64_t j = 0; j < G; j++)
            quant_group(W + n * K + j * g, g, sym, u + j * g, &scales[n * G + j],
                        &zp[j]);
        for (int64_t i = 0; i < K / 2; i++)
            codes[n * (K / 2) + i] = (uint8_t)(u[2 * i] | (u[2 * i + 1] << 4));
        if (!sym && zeros) {
            for (int64_t i = 0; i < Gz; i++) {
                int lo = zp[2 * i];
                int hi = (2 * i + 1 < G) ? zp[2 * i + 1] : 0;
                zeros[n * Gz + i] = (uint8_t)(lo | (hi << 4));
            }
        }
        free(zp);
        free(u);
    }
    return 0;
}

/* Dequantize rows [n0, n1) of a packed INT4 weight into fp64:
 * w_hat[n][k] = (u - zp) * s (Core ideas §2.2, dequantization), exact in
 * fp64. Symmetric weights (zeros == NULL) use zp = 8.                       */
void orc_q4_dequant_rows(const uint8_t *codes, const uint16_t *scales,
                         const uint8_t *zeros, int64_t K, int g, int64_t n0,
                         int64_t n1, double *out)
{
    int64_t G = K / g, Gz = (G + 1) / 2;
    for (int64_t n = n0; n < n1; n++) {
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte = codes[n * (K / 2) + k / 2];
            int u = (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);
            int64_t j = k / g;
            int zp = 8;
            if (zeros) {
                uint8_t zb = zeros[n * Gz + j / 2];
                zp = (j % 2 == 0) ? (zb & 0xf) : (zb >> 4);
            }
            double s = (double)orc_h2f(scales[n * G + j]);
            out[(n - n0) * K + k] = (double)(u - zp) * s;
        }
    }
}

/* W4A16 reference: Y[m][n] = sum_k x[m][k] * w_hat[n][k] in fp64 for the
 * listed rows m (all rows when rows == NULL), and the error scale
 * B[m][n] = sum_k |x| |w_hat|. Outputs are [n_rows, N]. The product is the
 * plain linear layer Y = X W^T over the dequantized weight (Quantization
 * operators guide §1.2: quantize, compute, dequantize).                    */
void orc_w4a16_ref(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes,
                   const uint16_t *scales, const uint8_t *zeros, int64_t N,
                   int g, const int64_t *rows, int64_t n_rows, double *Y,
                   double *B)
{
    (void)M;
    if (!rows) n_rows = M;
    double *xr = (double *)malloc(sizeof(double) * (size_t)(n_rows * K));
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; k++)
            xr[i * K + k] = (double)orc_h2f(X[m * K + k]);
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        orc_q4_dequant_rows(codes, scales, zeros, K, g, n, n + 1, w);
        for (int64_t i = 0; i < n_rows; i++) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t k = 0; k < K; k++) {
                acc += xr[i * K + k] * w[k];
                bnd += fabs(xr[i * K + k]) * fabs(w[k]);
            }
            Y[i * N + n] = acc;
            if (B) B[i * N + n] = bnd;
        }
        free(w);
    }
    free(xr);
}

/* ------------------------------------------------------------------------ */
/* AWQ-style per-input-channel scaling on the W4A16 path (Quantization
 * operators guide §3.2: W'' = W * s and x'' = x / s for every input channel;
 * Schemes notes, AWQ section: Y = X W = (X / s)(W * s)). The search for s is
 * offline; here s is given. Both operands stay binary16 (W4A16 keeps 16-bit
 * activations and quantizes 16-bit weights), so each scaled value is the
 * IEEE binary32 product or quotient, rounded once more to binary16:
 *   w''[n][k] = f2h(h2f(W[n][k]) * s[k])
 *   x''[m][k] = f2h(h2f(X[m][k]) / s[k])
 * The scaled layer is then the plain W4A16 product of x'' with the INT4
 * quantization of w'' (orc_q4_quantize_pack, orc_w4a16_ref).               */
void orc_awq_scale_weight(const uint16_t *W, const float *s, int64_t N, int64_t K,
                          uint16_t *Ws)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            float w = orc_h2f(W[n * K + k]) * s[k];
            Ws[n * K + k] = orc_f2h(w);
        }
}

void orc_awq_scale_act(const uint16_t *X, const float *s, int64_t M, int64_t K,
                       uint16_t *Xs)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++) {
            float x = orc_h2f(X[m * K + k]) / s[k];
            Xs[m * K + k] = orc_f2h(x);
        }
}

/* ------------------------------------------------------------------------ */
/* Per-channel INT8 weight with the SmoothQuant fold (Quantization operators
 * guide §2.2 per-channel: one scale per output row, max|w| / 127, codes
 * clamped to [-127, 127]; §5.1 and Core ideas §2.4: W' = W diag(s)).
 *   w'[n][k] = x * s[k]            (fp32 multiply; s == NULL means s = 1)
 *   a_n = max(max_k |w'|, 1e-8)    (the 1e-8 floor of the Method boundaries
 *                                   example's clamp_min)
 *   sw[n] = a_n / 127
 *   q = clip(rne(w' / sw[n]), -127, 127)
 * A row whose w' holds a NaN or an infinity is flagged: sw[n] = NaN, codes 0. */
void orc_q8_quantize_weight(const uint16_t *W, const float *s, int64_t N,
                            int64_t K, int8_t *Wq, float *sw)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float a = 0.0f;
        int bad = 0;
        for (int64_t k = 0; k < K; k++) {
            float w = orc_h2f(W[n * K + k]) * (s ? s[k] : 1.0f);
            if (!isfinite(w)) bad = 1;
            if (fabsf(w) > a) a = fabsf(w);
        }
        if (bad) {                              /* flagged row: NaN scale, codes 0 */
            for (int64_t k = 0; k < K; k++) Wq[n * K + k] = 0;
            sw[n] = NAN;
            continue;
        }
        if (a < 1e-8f) a = 1e-8f;
        float scale = a / 127.0f;
        for (int64_t k = 0; k < K; k++) {
            float w = orc_h2f(W[n * K + k]) * (s ? s[k] : 1.0f);
            int q = (int)rintf(w / scale);
            if (q < -127) q = -127;
            if (q > 127) q = 127;
            Wq[n * K + k] = (int8_t)q;
        }
        sw[n] = scale;
    }
}

/* Per-token dynamic INT8 activation quantization of the smoothed input
 * (Quantization schemes notes on per-token scales; Quantization operators
 * guide §5.1 transform X / s and §5.3 the online divide):
 *   x'[m][k] = x / s[k]            (fp32 division; s == NULL: x' = x)
 *   a_m = max(max_k |x'|, 1e-8),  sx[m] = a_m / 127,
 *   q = clip(rne(x' / sx[m]), -127, 127)
 * A row whose x' holds a NaN or an infinity is flagged: sx[m] = NaN, codes 0. */
void orc_q8_quantize_act(const uint16_t *X, const float *s, int64_t M,
                         int64_t K, int8_t *Xq, float *sx)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float a = 0.0f;
        int bad = 0;
        for (int64_t k = 0; k < K; k++) {
            float x = orc_h2f(X[m * K + k]);
            if (s) x = x / s[k];
            if (!isfinite(x)) bad = 1;
            if (fabsf(x) > a) a = fabsf(x);
        }
        if (bad) {                              /* flagged row: NaN scale, codes 0 */
            for (int64_t k = 0; k < K; k++) Xq[m * K + k] = 0;
            sx[m] = NAN;
            continue;
        }
        if (a < 1e-8f) a = 1e-8f;
        float scale = a / 127.0f;
        for (int64_t k = 0; k < K; k++) {
            float x = orc_h2f(X[m * K + k]);
            if (s) x = x / s[k];
            int q = (int)rintf(x / scale);
            if (q < -127) q = -127;
            if (q > 127) q = 127;
            Xq[m * K + k] = (int8_t)q;
        }
        sx[m] = scale;
    }
}

/* INT8 GEMM with exact integer accumulation (Quantization operators guide
 * §2.3: C_int32 = sum(A_int8 * B_int8); §5.2 path A: C = X_int8 W_int8^T).
 * acc[i][n] = sum_k Xq[m][k] * Wq[n][k] for the listed rows m (all when
 * rows == NULL), in int64; returns the number of results outside int32.     */
int64_t orc_int8_gemm(const int8_t *Xq, int64_t M, int64_t K, const int8_t *Wq,
                      int64_t N, const int64_t *rows, int64_t n_rows,
                      int64_t *acc, int64_t *abs_acc)
{
    if (!rows) n_rows = M;
    int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : overflow)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t i = 0; i < n_rows; i++) {
            int64_t m = rows ? rows[i] : i;
            int64_t a = 0, b = 0;
            for (int64_t k = 0; k < K; k++) {
                int64_t p = (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + k];
                a += p;
                b += p < 0 ? -p : p;
            }
            acc[i * N + n] = a;
            if (abs_acc) abs_acc[i * N + n] = b;
            if (a > INT32_MAX || a < INT32_MIN) overflow++;
        }
    }
    return overflow;
}

/* W8A8 epilogue (Quantization operators guide §2.3 DequantizeOp and §5.2:
 * C_fp16 = C_int32 * scale_X * scale_W).
 * Reference, fp64: Y = sx[m] * sw[n] * acc, B = sx[m] * sw[n] * sum|qx||qw|.
 * The same expression in fp32, ((float)acc * sx) * sw rounded once to fp16,
 * is returned in y16 (may be NULL).                                         */
void orc_w8a8_epilogue(const int64_t *acc, const int64_t *abs_acc,
                       const float *sx, const int64_t *rows, int64_t n_rows,
                       const float *sw, int64_t N, double *Y, double *B,
                       uint16_t *y16)
{
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; n++) {
            int64_t a = acc[i * N + n];
            Y[i * N + n] = (double)sx[m] * (double)sw[n] * (double)a;
            if (B) B[i * N + n] = (double)sx[m] * (double)sw[n] * (double)abs_acc[i * N + n];
            if (y16) {
                float f = (float)(int32_t)a;
                f = f * sx[m];
                f = f * sw[n];
                y16[i * N + n] = orc_f2h(f);
            }
        }
    }
}

/* SmoothQuant migration factor (Quantization operators guide §5.1; Core
 * ideas §2.4; Quantization notes, SmoothQuant):
 *   s_j = max|X_j|^alpha / max|W_j|^(1 - alpha),
 * with X the calibration activations [R, K] and W the weight [N, K]; the
 * weight maximum for input channel j is taken over the output rows. Both
 * maxima are floored at 1e-8. At alpha = 0.5 the powers are square roots,
 * computed with the correctly rounded sqrtf.                               */
void orc_smooth_scales(const uint16_t *Xcal, int64_t R, const uint16_t *W,
                       int64_t N, int64_t K, float alpha, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; j++) {
        float ax = 0.0f, aw = 0.0f;
        for (int64_t r = 0; r < R; r++) {
            float v = fabsf(orc_h2f(Xcal[r * K + j]));
            if (v > ax) ax = v;
        }
        for (int64_t n = 0; n < N; n++) {
            float v = fabsf(orc_h2f(W[n * K + j]));
            if (v > aw) aw = v;
        }
        if (ax < 1e-8f) ax = 1e-8f;
        if (aw < 1e-8f) aw = 1e-8f;
        if (alpha == 0.5f)
            s[j] = sqrtf(ax) / sqrtf(aw);
        else
            s[j] = powf(ax, alpha) / powf(aw, 1.0f - alpha);
    }
}

/* ------------------------------------------------------------------------ */
/* Small-float decoders written from the format definitions (Core ideas
 * §2.1: E4M3 = 1+4+3 with S.1111.111 as NaN, E5M2 = 1+5+2 IEEE-style with
 * the all-ones exponent for Inf/NaN, E2M1 = 1+2+1). Exponent bias is
 * 2^(e-1) - 1; exponent field 0 is subnormal (no implicit 1).               */
static float decode_minifloat(unsigned code, int ebits, int mbits, int ieee_specials,
                              int nan_all_ones)
{
    unsigned sign = (code >> (ebits + mbits)) & 1;
    unsigned e = (code >> mbits) & ((1u << ebits) - 1);
    unsigned m = code & ((1u << mbits) - 1);
    unsigned emax = (1u << ebits) - 1;
    int bias = (1 << (ebits - 1)) - 1;
    float v;
    if (ieee_specials && e == emax)
        v = m ? NAN : INFINITY;
    else if (nan_all_ones && e == emax && m == (1u << mbits) - 1)
        v = NAN;
    else if (e == 0)
        v = ldexpf((float)m, 1 - bias - mbits);
    else
        v = ldexpf((float)((1u << mbits) + m), (int)e - bias - mbits);
    return sign ? -v : v;
}

float orc_e4m3_decode(unsigned code) { return decode_minifloat(code & 0xff, 4, 3, 0, 1); }
float orc_e5m2_decode(unsigned code) { return decode_minifloat(code & 0xff, 5, 2, 1, 0); }
float orc_e2m1_decode(unsigned code) { return decode_minifloat(code & 0xf, 2, 1, 0, 0); }

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 path (Quantization operators guide §4.1 formats, §4.2 scaled FP8
 * GEMM: C = scale_A * scale_B * (A_fp8 @ B_fp8); Core ideas §2.1 E4M3 range
 * +-448). Weights and activations both in E4M3, scaled per output channel
 * and per token like the INT8 path, with 448 in place of 127.               */

/* Nearest E4M3 value to x, ties to the even mantissa, saturating at +-448
 * (the guide clamps to the format maximum before the cast), sign kept on
 * zero. Written from the format: bias 7, three mantissa bits, exponent field
 * 0 holds the subnormals m * 2^-9, the largest finite value is 1.75 * 2^8.  */
unsigned orc_e4m3_encode(float x)
{
    unsigned sign = signbit(x) ? 0x80u : 0u;
    float a = fabsf(x);
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < ldexpf(1.0f, -6)) {                 /* subnormal range: quantum 2^-9 */
        int q = (int)rintf(ldexpf(a, 9));       /* exact scaling, RNE */
        return sign | (unsigned)q;              /* q == 8 is the smallest normal, 0x08 */
    }
    int e;
    frexpf(a, &e);                              /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                                     /* a in [2^e, 2^(e+1)) */
    int q = (int)rintf(ldexpf(a, 3 - e));       /* 8 .. 16: mantissa with the implicit 1 */
    if (q == 16) {
        q = 8;
        e += 1;
    }
    unsigned code = (unsigned)((e + 7) << 3) | (unsigned)(q - 8);
    if (code > 0x7Eu) code = 0x7Eu;             /* rounding up past 448 saturates */
    return sign | code;
}

/* One row of the FP8 quantizer: v[k] = x * s[k] (weight, mul != 0) or
 * x / s[k] (activation), a = max(max_k |v|, 1e-8), scale = a / 448,
 * q[k] = e4m3(v[k] / scale). A row whose v holds a NaN or an infinity is
 * flagged: scale NaN, codes 0.                                              */
static void fp8_row(const uint16_t *x, const float *s, int64_t K, int mul, uint8_t *q,
                    float *scale_out)
{
    float a = 0.0f;
    int bad = 0;
    for (int64_t k = 0; k < K; k++) {
        float v = orc_h2f(x[k]);
        if (s) v = mul ? v * s[k] : v / s[k];
        if (!isfinite(v)) bad = 1;
        if (fabsf(v) > a) a = fabsf(v);
    }
    if (bad) {                                  /* flagged row: NaN scale, codes 0 */
        for (int64_t k = 0; k < K; k++) q[k] = 0;
        *scale_out = NAN;
        return;
    }
    if (a < 1e-8f) a = 1e-8f;
    float scale = a / 448.0f;
    for (int64_t k = 0; k < K; k++) {
        float v = orc_h2f(x[k]);
        if (s) v = mul ? v * s[k] : v / s[k];
        q[k] = (uint8_t)orc_e4m3_encode(v / scale);
    }
    *scale_out = scale;
}

/* Per-output-channel E4M3 weight of W diag(s) (s == NULL: s = 1). */
void orc_fp8_quantize_weight(const uint16_t *W, const float *s, int64_t N, int64_t K,
                             uint8_t *Wq, float *sw)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) fp8_row(W + n * K, s, K, 1, Wq + n * K, sw + n);
}

/* Per-token dynamic E4M3 activation of X / s (s == NULL: X as is). */
void orc_fp8_quantize_act(const uint16_t *X, const float *s, int64_t M, int64_t K,
                          uint8_t *Xq, float *sx)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) fp8_row(X + m * K, s, K, 0, Xq + m * K, sx + m);
}

/* FP8 GEMM reference: acc[i][n] = sum_k e4m3(Xq[m][k]) * e4m3(Wq[n][k]) for
 * the listed rows (all when rows == NULL), and sum_k |product|. Each product
 * is a multiple of 2^-18 below 2^18, so K <= 2^16 of them sum exactly in
 * fp64: the reference is the exact sum.                                      */
void orc_fp8_gemm(const uint8_t *Xq, int64_t M, int64_t K, const uint8_t *Wq, int64_t N,
                  const int64_t *rows, int64_t n_rows, double *acc, double *abs_acc)
{
    if (!rows) n_rows = M;
    float lut[256];
    for (int c = 0; c < 256; c++) lut[c] = orc_e4m3_decode((unsigned)c);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t i = 0; i < n_rows; i++) {
            int64_t m = rows ? rows[i] : i;
            double a = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)lut[Xq[m * K + k]] * (double)lut[Wq[n * K + k]];
                a += p;
                b += fabs(p);
            }
            acc[i * N + n] = a;
            abs_acc[i * N + n] = b;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP4 weights (Quantization operators guide §4.3: FP4 E2M1 elements, one
 * E8M0 scale per block of 32; weights in FP4, activations kept in FP8; the
 * Schemes notes list the E2M1 value set {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4,
 * +-6}).                                                                      */

/* Nearest E2M1 value to x, ties to the even mantissa, saturating at +-6,
 * sign kept on zero. Codes: sign bit 3, exponent bits 2-1 (bias 1), mantissa
 * bit 0; exponent 0 is the subnormal 0.5 * m.                               */
unsigned orc_e2m1_encode(float x)
{
    unsigned sign = signbit(x) ? 0x8u : 0u;
    float a = fabsf(x);
    if (a >= 6.0f) return sign | 0x7u;
    if (a < 1.0f) return sign | (unsigned)rintf(a * 2.0f);   /* 0, 0.5, 1.0 (code 2) */
    int e;
    frexpf(a, &e);
    e -= 1;                                                   /* a in [2^e, 2^(e+1)), e in 0..2 */
    int q = (int)rintf(ldexpf(a, 1 - e));                     /* 2 or 3; 4 carries */
    if (q == 4) {
        q = 2;
        e += 1;
    }
    unsigned code = (unsigned)((e + 1) << 1) | (unsigned)(q - 2);
    if (code > 0x7u) code = 0x7u;
    return sign | code;
}

/* MXFP4 quantizer of W diag(s) (s == NULL: s = 1), block of 32 along K:
 *   v = w * s[k] (fp32), amax = max over the block of |v|,
 *   scale = 2^(e - 127) with e the smallest integer such that amax <= 6 * 2^(e - 127)
 *           (the smallest power of two that keeps every element in range;
 *           e = 0 for an all-zero block; e <= 254),
 *   code  = e2m1(v / scale) (exact division by a power of two);
 * a block whose v holds a NaN or an infinity is flagged: scale byte 0xff
 * (E8M0's NaN), codes 0.
 * Codes packed two per byte along K (even k in the low nibble) [N, K/2];
 * scales E8M0 bytes [N, K/32].                                               */
void orc_mxfp4_quantize_weight(const uint16_t *W, const float *s, int64_t N, int64_t K,
                               uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            float v[32], amax = 0.0f;
            int bad = 0;
            for (int i = 0; i < 32; i++) {
                int64_t k = b * 32 + i;
                v[i] = orc_h2f(W[n * K + k]) * (s ? s[k] : 1.0f);
                if (!isfinite(v[i])) bad = 1;
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            if (bad) {                          /* flagged block: E8M0 NaN 0xff, codes 0 */
                scales[n * nb + b] = 0xff;
                for (int i = 0; i < 16; i++) codes[n * (K / 2) + b * 16 + i] = 0;
                continue;
            }
            int e = 0;
            if (amax > 0.0f) {
                e = 1;
                while (e < 254 && amax > 6.0f * ldexpf(1.0f, e - 127)) e++;
                /* ldexpf(1, e - 127) is the subnormal 2^-126 at e = 1, exact */
            }
            scales[n * nb + b] = (uint8_t)e;
            for (int i = 0; i < 32; i += 2) {
                unsigned lo = orc_e2m1_encode(ldexpf(v[i], 127 - e));
                unsigned hi = orc_e2m1_encode(ldexpf(v[i + 1], 127 - e));
                codes[n * (K / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* W4A8 reference: acc[i][n] = sum_k e4m3(Xq[m][k]) * e2m1(W[n][k]) * 2^(e[n][k/32] - 127)
 * for the listed rows m, and the sum of |products|, in fp64 (exact while the
 * block exponents of a row span fewer than about 30 binades).                 */
void orc_mxfp4_gemm(const uint8_t *Xq, int64_t M, int64_t K, const uint8_t *codes,
                    const uint8_t *scales, int64_t N, const int64_t *rows, int64_t n_rows,
                    double *acc, double *abs_acc)
{
    if (!rows) n_rows = M;
    float lut8[256], lut4[16];
    for (int c = 0; c < 256; c++) lut8[c] = orc_e4m3_decode((unsigned)c);
    for (int c = 0; c < 16; c++) lut4[c] = orc_e2m1_decode((unsigned)c);
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t i = 0; i < n_rows; i++) {
            int64_t m = rows ? rows[i] : i;
            double a = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; k++) {
                uint8_t byte = codes[n * (K / 2) + k / 2];
                unsigned c4 = (k & 1) ? (byte >> 4) : (byte & 0xFu);
                double w = ldexp((double)lut4[c4], (int)scales[n * nb + k / 32] - 127);
                double p = (double)lut8[Xq[m * K + k]] * w;
                a += p;
                b += fabs(p);
            }
            acc[i * N + n] = a;
            abs_acc[i * N + n] = b;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* NF4 weights (Quantization operators guide §3.4: 16 non-uniform levels, the
 * medians of 16 equal-probability intervals of N(0, 1) normalised to
 * [-1, 1] and stored in fp16; per block of 64 weights one fp32 scale, the
 * block's max |w|; code = index of the nearest level to w / scale).
 * The level table is an input (fp16 bit patterns, ascending), so the
 * quantile function stays with its library.                                  */

/* codes [N, K/2] (two per byte along K, even k in the low nibble), scales
 * fp32 [N, K/64]: scale = max(max_block |w|, 1e-8), x = w / scale (fp32
 * IEEE), code = the first index i minimising fabsf(x - level[i]) (fp32).
 * A block holding a NaN or an infinity is flagged: scale NaN, codes 0.      */
void orc_nf4_quantize(const uint16_t *W, int64_t N, int64_t K, const uint16_t *levels,
                      uint8_t *codes, float *scales)
{
    float lv[16];
    for (int i = 0; i < 16; i++) lv[i] = orc_h2f(levels[i]);
    const int64_t nb = K / 64;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            float a = 0.0f;
            int bad = 0;
            for (int i = 0; i < 64; i++) {
                float v = fabsf(orc_h2f(W[n * K + b * 64 + i]));
                if (!isfinite(v)) bad = 1;
                if (v > a) a = v;
            }
            if (bad) {                          /* flagged block: NaN scale, codes 0 */
                scales[n * nb + b] = NAN;
                for (int i = 0; i < 32; i++) codes[n * (K / 2) + b * 32 + i] = 0;
                continue;
            }
            if (a < 1e-8f) a = 1e-8f;
            scales[n * nb + b] = a;
            for (int i = 0; i < 64; i++) {
                float x = orc_h2f(W[n * K + b * 64 + i]) / a;
                int best = 0;
                float bd = fabsf(x - lv[0]);
                for (int l = 1; l < 16; l++) {
                    float d = fabsf(x - lv[l]);
                    if (d < bd) {
                        bd = d;
                        best = l;
                    }
                }
                int64_t k = b * 64 + i;
                uint8_t *byte = &codes[n * (K / 2) + k / 2];
                if (k & 1) *byte = (uint8_t)((*byte & 0x0F) | (best << 4));
                else *byte = (uint8_t)((*byte & 0xF0) | best);
            }
        }
    }
}

/* fp64 reference of Y = X W_hat^T with w_hat = level[code] * scale (exact in
 * fp64), and B = sum |x| |w_hat|, for the listed rows of X.                 */
void orc_nf4_ref(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes,
                 const float *scales, const uint16_t *levels, int64_t N,
                 const int64_t *rows, int64_t n_rows, double *Y, double *B)
{
    if (!rows) n_rows = M;
    double lv[16];
    for (int i = 0; i < 16; i++) lv[i] = (double)orc_h2f(levels[i]);
    const int64_t nb = K / 64;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t i = 0; i < n_rows; i++) {
            int64_t m = rows ? rows[i] : i;
            double y = 0.0, bb = 0.0;
            for (int64_t k = 0; k < K; k++) {
                uint8_t byte = codes[n * (K / 2) + k / 2];
                int c = (k & 1) ? (byte >> 4) : (byte & 0xF);
                double w = lv[c] * (double)scales[n * nb + k / 64];
                double x = (double)orc_h2f(X[m * K + k]);
                y += x * w;
                bb += fabs(x) * fabs(w);
            }
            Y[i * N + n] = y;
            B[i * N + n] = bb;
        }
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif

/* ------------------------------------------------------------------------ */
/* NVFP4 weights (Quantization notes, FP4 item: FP4 E2M1 values with one FP8
 * scale per block of 16 (4 + 8/16 = 4.5 bits per weight); its NVFP4-style
 * sketch takes the block's max |w|, the scale amax / 6 cast to FP8 E4M3, and
 * the FP4 value of w / scale clipped to +-6). The sketch's line that rounds
 * w / scale * 6 to an integer is read as what the rest of the item says: the
 * E2M1 value of w / scale.
 *   scale = e4m3(fl32(amax / 6))   (nearest, ties to even, saturating at 448)
 *   code  = e2m1(fl32(w / scale))  (nearest, ties to even, saturating at 6);
 *           every code of a block whose scale is 0 (amax / 6 at most 2^-10,
 *           half the smallest E4M3 subnormal) is 0
 *   w_hat = e2m1(code) * e4m3(scale)
 * A block holding a NaN or an infinity is flagged: scale byte 0x7f (E4M3's
 * NaN), codes 0.
 * Codes [N, K/2] (two per byte along K, even k in the low nibble), scales
 * E4M3 bytes [N, K/16].                                                      */
void orc_nvfp4_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            float v[16], amax = 0.0f;
            int bad = 0;
            for (int i = 0; i < 16; i++) {
                v[i] = orc_h2f(W[n * K + b * 16 + i]);
                if (!isfinite(v[i])) bad = 1;
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            if (bad) {                          /* flagged block: E4M3 NaN 0x7f, codes 0 */
                scales[n * nb + b] = 0x7f;
                for (int i = 0; i < 8; i++) codes[n * (K / 2) + b * 8 + i] = 0;
                continue;
            }
            const unsigned sc = orc_e4m3_encode(amax / 6.0f);
            const float scale = orc_e4m3_decode(sc);
            scales[n * nb + b] = (uint8_t)sc;
            for (int i = 0; i < 16; i += 2) {
                unsigned lo = 0, hi = 0;
                if (scale > 0.0f) {
                    lo = orc_e2m1_encode(v[i] / scale);
                    hi = orc_e2m1_encode(v[i + 1] / scale);
                }
                codes[n * (K / 2) + b * 8 + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* Y = X W_hat^T and B = |X| |W_hat|^T in fp64 for the listed rows of X (all
 * when rows == NULL), w_hat = e2m1(code) * e4m3(scale of its block of 16).   */
void orc_nvfp4_ref(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes,
                   const uint8_t *scales, int64_t N, const int64_t *rows, int64_t n_rows,
                   double *Y, double *B)
{
    if (!rows) n_rows = M;
    const int64_t nb = K / 16;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t i = 0; i < n_rows; i++) {
            int64_t m = rows ? rows[i] : i;
            double y = 0.0, bb = 0.0;
            for (int64_t k = 0; k < K; k++) {
                uint8_t byte = codes[n * (K / 2) + k / 2];
                unsigned c = (k & 1) ? (byte >> 4) : (byte & 0xFu);
                double w = (double)orc_e2m1_decode(c) * (double)orc_e4m3_decode(scales[n * nb + k / 16]);
                double x = (double)orc_h2f(X[m * K + k]);
                y += x * w;
                bb += fabs(x) * fabs(w);
            }
            Y[i * N + n] = y;
            B[i * N + n] = bb;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* LayerNorm, the SmoothQuant divide and the per-token INT8 quantizer as one
 * operation (Quantization operators guide §5.3, deployment fusion: the
 * online X / s is folded into the epilogue of the LayerNorm that produces
 * the activations, and its output is quantized straight away; Method
 * boundaries, SmoothQuant section: the scale may be folded into the
 * preceding norm). For each row x of X (fp16, length K):
 *   S1 = sum_k x_k, S2 = sum_k x_k^2          (exact: fp16 values are
 *        integer multiples of 2^-24, so the sums are taken on the integers
 *        a_k = x_k 2^24, S1 in int64, S2 in a 128-bit integer)
 *   mean = fl64(S1) / K                       (fp64, one rounding)
 *   ex2  = fl64(S2) / K                       (S2 rounded once to fp64)
 *   var  = max(ex2 - mean * mean, 0)          (fp64; the biased variance of
 *                                              LayerNorm)
 *   r    = 1 / sqrt(var + eps)                (fp64, correctly rounded)
 *   g_k  = gamma_k / s_k, b_k = beta_k / s_k  (fp64 divisions of the fp32
 *        parameters: the divide by s folded into the affine step; s == NULL
 *        means s = 1)
 *   x'_k = fl32(fma((x_k - mean) * r, g_k, b_k))
 * then the per-token quantizer of orc_q8_quantize_act on x':
 *   a = max(max_k |x'_k|, 1e-8), sx = a / 127 (fp32),
 *   q_k = clip(rne(x'_k / sx), -127, 127)     (fp32 division).
 * A row holding a non-finite x_k, or whose x' is not finite, is flagged:
 * sx = NaN, codes 0. eps must be positive. Optional outputs: xs [M, K] (x'),
 * stats [M, 3] (mean, var, r).                                              */
static int64_t half_units(uint16_t h)   /* h * 2^24 for a finite fp16 h */
{
    int e = (h >> 10) & 0x1f;
    int64_t f = h & 0x3ff;
    int64_t a = e ? (1024 + f) << (e - 1) : f;
    return (h >> 15) ? -a : a;
}

/* The LayerNorm part for one row: x' into xp, the statistics into st (mean,
 * var, r; NaN for a row with a non-finite x); returns 1 when the row is
 * flagged (a non-finite x or x').                                          */
static int ln_row(const uint16_t *x, const float *gamma, const float *beta, const float *s,
                  double eps, int64_t K, float *xp, double *st)
{
    int bad = 0;
    for (int64_t k = 0; k < K; k++)
        if (!isfinite(orc_h2f(x[k]))) bad = 1;
    double mean = NAN, var = NAN, r = NAN;
    if (!bad) {
        int64_t s1 = 0;
        unsigned __int128 s2 = 0;
        for (int64_t k = 0; k < K; k++) {
            int64_t a = half_units(x[k]);
            s1 += a;
            s2 += (unsigned __int128)(a < 0 ? -a : a) * (unsigned __int128)(a < 0 ? -a : a);
        }
        mean = ldexp((double)s1, -24) / (double)K;
        double ex2 = ldexp((double)s2, -48) / (double)K;
        double mm = mean * mean;
        var = ex2 - mm;
        if (var < 0.0) var = 0.0;
        double sd = sqrt(var + eps);
        r = 1.0 / sd;
        for (int64_t k = 0; k < K; k++) {
            double sk = s ? (double)s[k] : 1.0;
            double g = (double)gamma[k] / sk;
            double b = (double)beta[k] / sk;
            double d = (double)orc_h2f(x[k]) - mean;
            double nk = d * r;
            xp[k] = (float)fma(nk, g, b);
            if (!isfinite(xp[k])) bad = 1;
        }
    }
    if (st) {
        st[0] = mean;
        st[1] = var;
        st[2] = r;
    }
    return bad;
}

void orc_layernorm_quant_smooth(const uint16_t *X, const float *gamma, const float *beta,
                                const float *s, double eps, int64_t M, int64_t K,
                                int8_t *Xq, float *sx, float *xs, double *stats)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float *xp = xs ? xs + m * K : (float *)malloc((size_t)K * sizeof(float));
        int bad = ln_row(X + m * K, gamma, beta, s, eps, K, xp, stats ? stats + 3 * m : NULL);
        if (bad) {                              /* flagged row: NaN scale, codes 0 */
            for (int64_t k = 0; k < K; k++) {
                Xq[m * K + k] = 0;
                if (xs) xp[k] = NAN;
            }
            sx[m] = NAN;
        } else {
            float a = 0.0f;
            for (int64_t k = 0; k < K; k++)
                if (fabsf(xp[k]) > a) a = fabsf(xp[k]);
            if (a < 1e-8f) a = 1e-8f;
            float scale = a / 127.0f;
            for (int64_t k = 0; k < K; k++) {
                int q = (int)rintf(xp[k] / scale);
                if (q < -127) q = -127;
                if (q > 127) q = 127;
                Xq[m * K + k] = (int8_t)q;
            }
            sx[m] = scale;
        }
        if (!xs) free(xp);
    }
}

/* The same LayerNorm with the FP8 E4M3 per-token quantizer of
 * orc_fp8_quantize_act in place of the INT8 one (the FP8 variant of the
 * path): scale = max(max_k |x'|, 1e-8) / 448, codes e4m3(x' / scale).       */
void orc_layernorm_quant_smooth_fp8(const uint16_t *X, const float *gamma, const float *beta,
                                    const float *s, double eps, int64_t M, int64_t K,
                                    uint8_t *Xq, float *sx)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float *xp = (float *)malloc((size_t)K * sizeof(float));
        if (ln_row(X + m * K, gamma, beta, s, eps, K, xp, NULL)) {
            for (int64_t k = 0; k < K; k++) Xq[m * K + k] = 0;
            sx[m] = NAN;
        } else {
            float a = 0.0f;
            for (int64_t k = 0; k < K; k++)
                if (fabsf(xp[k]) > a) a = fabsf(xp[k]);
            if (a < 1e-8f) a = 1e-8f;
            float scale = a / 448.0f;
            for (int64_t k = 0; k < K; k++) Xq[m * K + k] = (uint8_t)orc_e4m3_encode(xp[k] / scale);
            sx[m] = scale;
        }
        free(xp);
    }
}

/* The fp64 value of an unsigned 128-bit integer hi 2^64 + lo, as the cast
 * above rounds it (exposed so the tests can check that rounding against an
 * independent one).                                                        */
double orc_u128_to_double(uint64_t hi, uint64_t lo)
{
    unsigned __int128 v = ((unsigned __int128)hi << 64) | lo;
    return (double)v;
}
