/*
 * w4a8_oracle.c -- plain CPU oracle for the W4A8 progressive-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code, header or table with the
 * GPU kernels.
 *
 * It computes, step by step and in the most direct form, what the method
 * defines:
 *
 *   Y[M,N] = X[M,K] . W[N,K]^T
 *
 * with W progressively quantized (per-output-channel symmetric INT8 inside a
 * protective range, then per-group-of-128 asymmetric UINT4 with an integer
 * scale and a zero point), X quantized per token to INT8 by its absolute
 * maximum, an exact integer contraction (int64 accumulation, stored as int32),
 * and an fp32 epilogue that applies the two scales and rounds to fp16.
 *
 * Sources (pages, by title):
 *  - "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 *    Serving" (MLSys'25 talk summary), sections "Progressive Group Quantization
 *    for W4A8 GEMM", "Quantized Matrix Multiplication (GEMM) Kernel on GPUs",
 *    "Challenges and Design Details of QServe GEMM Kernel".
 *  - Lecture 15 notes (cs2680), section 15.6 "QServe: W4A8KV4, and paying for
 *    dequant once".
 *  - "QFactory: Accelerating Quantized Large Language Model Serving with Qtile
 *    Graphs" (reading notes), section 2.1 (asymmetric quantization and its
 *    dequantization w = (w_quant - zero) * scale).
 *
 * Where the pages leave a rounding or tie rule open, the reading used here is
 * written next to the step.  All floating-point steps are IEEE fp32 with
 * round-to-nearest-even; build with -ffp-contract=off so no FMA is formed.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void);

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 conversions, written from the format's definition:     */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have  */
/* value frac * 2^-24.                                                       */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> float (exact: every binary16 value is a float). */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* float -> binary16 bits, round to nearest, ties to even.
 * Every float is exactly representable in double, and scaling by a power of
 * two is exact, so rint() on the scaled value takes the rounding decision on
 * the exact value. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    /* The largest finite binary16 is 65504; the midpoint to the next binade
     * (65536, which overflows) is 65520, and the tie goes to the even
     * neighbour, i.e. to infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24 (may round up to the
         * smallest normal, 1024 * 2^-24, whose bit pattern is 0x0400) */
        double n = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2);            /* a = m * 2^e2 with m in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)) */
    double n = rint(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)n - 1024));
}

/* ------------------------------------------------------------------------ */
/* Integer division rounded to nearest, ties to even (d > 0).               */
/* ------------------------------------------------------------------------ */
int64_t orc_rne_div(int64_t p, int64_t d)
{
    int64_t q = p / d;
    int64_t r = p % d;
    if (r < 0) {              /* make q = floor(p / d), r in [0, d) */
        q -= 1;
        r += d;
    }
    if (2 * r > d)
        q += 1;
    else if (2 * r == d)
        q += (q & 1);         /* exact half: go to the even quotient */
    return q;
}

static float clampf(float v, float lo, float hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

static int64_t clampi(int64_t v, int64_t lo, int64_t hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

/* ------------------------------------------------------------------------ */
/* Activations: per-token symmetric INT8 by absolute maximum.               */
/* The QServe talk summary ("Precision Data Flow and Activation             */
/* Quantization Fusion") makes every linear layer take 8-bit inputs; the    */
/* per-token absmax rule with 127 levels per side is the method's stated   */
/* activation quantizer.  Readings: fp32 scale a/127 by IEEE division,      */
/* code = rint(x / scale) (ties to even), clamped to [-127, 127]; an        */
/* all-zero token gets scale 0 and all-zero codes.                          */
/* x is fp16 bits, row stride ldx elements.                                 */
/* ------------------------------------------------------------------------ */
void orc_quantize_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                      int8_t *qx, float *s_a)
{
    for (int64_t m = 0; m < M; m++) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float v = fabsf(orc_f16_to_f32(x[m * ldx + k]));
            if (v > a)
                a = v;
        }
        float s = a / 127.0f;
        s_a[m] = s;
        for (int64_t k = 0; k < K; k++) {
            float q = 0.0f;
            if (a != 0.0f) {
                float t = orc_f16_to_f32(x[m * ldx + k]) / s;
                q = clampf(rintf(t), -127.0f, 127.0f);
            }
            qx[m * K + k] = (int8_t)q;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Normalization fused with the activation quantizer.  The QServe talk      */
/* summary ("Precision Data Flow and Activation Quantization Fusion") has   */
/* the layer before a linear layer -- its example is LayerNorm -- emit the  */
/* 8-bit activations directly.  Per token m, over its K features:           */
/*   LayerNorm (rms == 0): h = (x - mean) / sqrt(var + eps) * gamma + beta  */
/*   RMSNorm   (rms != 0): h = x / sqrt(mean(x^2) + eps) * gamma (+ beta)   */
/* and the fp16 row h is quantized by orc_quantize_act's rule.  The pages   */
/* give no precision for the statistics; the readings:                      */
/*   - mean is exact up to one rounding: an fp16 value is an integer       */
/*     multiple of 2^-24, so the row sum is an exact integer S and          */
/*     mean = (double(S) * 2^-24) / K (IEEE double; 0 for RMSNorm);         */
/*   - var = (sum over k, in order, of (double(x) - mean)^2) / K in double, */
/*     each product and sum rounded (x^2 for RMSNorm);                      */
/*   - r = 1 / sqrt(var + eps) in double (IEEE sqrt and division); the fp32 */
/*     factors are mean32 = float(mean) and rstd = float(r), with rstd = 0  */
/*     when var + eps is 0;                                                  */
/*   - h = fp16( ((float(x) - mean32) * rstd) * float(gamma) + float(beta)) */
/*     in fp32 in that order (no beta: no addition).                         */
/* The sum of squares is the one step whose rounding depends on the order   */
/* of the additions; an implementation that adds in another order gets a    */
/* double r within about K * 2^-53 of this one, and the same rstd unless r  */
/* lies that close to a midpoint between two floats.                        */
/* mean_out and r_out (double [M]) may be NULL; h (fp16 bits [M, K]) may be  */
/* NULL.  K <= 2^20 keeps S inside int64.                                    */
/* ------------------------------------------------------------------------ */
void orc_norm_quantize_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                           const uint16_t *gamma, const uint16_t *beta, float eps, int rms,
                           int8_t *qx, float *s_a, uint16_t *h, double *mean_out,
                           double *r_out)
{
    uint16_t *row = (uint16_t *)malloc((size_t)K * sizeof(uint16_t));
    for (int64_t m = 0; m < M; m++) {
        const uint16_t *xm = x + m * ldx;
        double mean = 0.0;
        if (!rms) {
            int64_t S = 0;
            for (int64_t k = 0; k < K; k++)
                S += (int64_t)ldexp((double)orc_f16_to_f32(xm[k]), 24);   /* exact integer */
            mean = ldexp((double)S, -24) / (double)K;
        }
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double d = (double)orc_f16_to_f32(xm[k]) - mean;
            double sq = d * d;
            ss = ss + sq;
        }
        double var = ss / (double)K;
        double ve = var + (double)eps;
        double r = ve == 0.0 ? INFINITY : 1.0 / sqrt(ve);
        float rstd = ve == 0.0 ? 0.0f : (float)r;
        float mean32 = (float)mean;
        if (mean_out)
            mean_out[m] = mean;
        if (r_out)
            r_out[m] = r;
        for (int64_t k = 0; k < K; k++) {
            float t = orc_f16_to_f32(xm[k]) - mean32;
            t = t * rstd;
            t = t * orc_f16_to_f32(gamma[k]);
            if (beta)
                t = t + orc_f16_to_f32(beta[k]);
            row[k] = orc_f32_to_f16(t);
        }
        if (h)
            memcpy(h + m * K, row, (size_t)K * sizeof(uint16_t));
        orc_quantize_act(row, 1, K, K, qx + m * K, s_a + m);
    }
    free(row);
}

/* ------------------------------------------------------------------------ */
/* Weights, level 1: per output channel, symmetric INT8 inside the          */
/* protective range [-119, 119], with an fp16 scale (QServe talk summary,   */
/* "Progressive Group Quantization for W4A8 GEMM"; Lecture 15 notes, 15.6,  */
/* level 1 of the two-level scheme: int8 envelope, fp16 channel scales).    */
/* Readings: s0 = fp16(absmax / 119) (fp32 division, then RNE to fp16);     */
/* codes divide by the stored fp16 value; rint ties to even; a zero row     */
/* has s0 = 0 and zero codes.                                               */
/* ------------------------------------------------------------------------ */
#define ORC_PROTECT 119

void orc_weights_level1(const float *w, int64_t N, int64_t K,
                        int8_t *q8, uint16_t *s0)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float v = fabsf(w[n * K + k]);
            if (v > a)
                a = v;
        }
        uint16_t h = orc_f32_to_f16(a / (float)ORC_PROTECT);
        s0[n] = h;
        float s = orc_f16_to_f32(h);
        for (int64_t k = 0; k < K; k++) {
            float q = 0.0f;
            if (s != 0.0f)
                q = clampf(rintf(w[n * K + k] / s), -(float)ORC_PROTECT,
                           (float)ORC_PROTECT);
            q8[n * K + k] = (int8_t)q;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Weights, level 2: per group of 128 consecutive k in one output row,      */
/* asymmetric UINT4 with an integer scale s1 and a zero point z             */
/* (QServe talk summary, "Progressive Group Quantization for W4A8 GEMM":    */
/* INT8 -> INT4 per group; Lecture 15 notes, 15.6: int8 scales per g=128    */
/* group; QFactory notes 2.1: min and max map to the ends of the integer    */
/* range).  All integer arithmetic.  Readings:                              */
/*   lo = min(0, min q8), hi = max(0, max q8)   (range contains 0, so the  */
/*                                              zero point is in [0, 15])  */
/*   s1 = max(1, ceil((hi - lo) / 15))          (integer scale covering the */
/*                                              whole range)               */
/*   z  = rne(-lo / s1)                                                     */
/*   q4 = clamp(rne(q8 / s1) + z, 0, 15)                                    */
/* q4 is returned one code per byte, [N, K]; s1, z are [N, K/128].          */
/* ------------------------------------------------------------------------ */
#define ORC_GROUP 128

void orc_weights_level2(const int8_t *q8, int64_t N, int64_t K,
                        uint8_t *q4, uint8_t *s1, uint8_t *z)
{
    int64_t G = K / ORC_GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t g = 0; g < G; g++) {
            const int8_t *src = q8 + n * K + g * ORC_GROUP;
            int64_t lo = 0, hi = 0;
            for (int64_t i = 0; i < ORC_GROUP; i++) {
                if (src[i] < lo)
                    lo = src[i];
                if (src[i] > hi)
                    hi = src[i];
            }
            int64_t D = hi - lo;
            int64_t s = (D + 14) / 15;          /* ceil(D / 15) */
            if (s < 1)
                s = 1;
            int64_t zz = orc_rne_div(-lo, s);
            s1[n * G + g] = (uint8_t)s;
            z[n * G + g] = (uint8_t)zz;
            for (int64_t i = 0; i < ORC_GROUP; i++) {
                int64_t c = clampi(orc_rne_div(src[i], s) + zz, 0, 15);
                q4[n * K + g * ORC_GROUP + i] = (uint8_t)c;
            }
        }
    }
}

/* Canonical packed form: [N, K/2] bytes, k even in the low nibble. */
void orc_pack_q4(const uint8_t *q4, int64_t N, int64_t K, uint8_t *packed)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k += 2)
            packed[n * (K / 2) + k / 2] =
                (uint8_t)((q4[n * K + k] & 0xF) | ((q4[n * K + k + 1] & 0xF) << 4));
}

/* ------------------------------------------------------------------------ */
/* Dequantization UINT4 -> INT8 by subtraction after multiplication         */
/* (QServe talk summary, "Challenges and Design Details of QServe GEMM      */
/* Kernel": multiply by the scale, then subtract the precomputed            */
/* zero*scale; Lecture 15 notes, 15.6).  Equal, as integers, to             */
/* (q4 - z) * s1 (QFactory notes 2.1).                                       */
/* Returns the number of reconstructions outside [-127, 127] or with       */
/* q4*s1 or z*s1 above 240 (0 when the protective range holds).            */
/* ------------------------------------------------------------------------ */
int64_t orc_dequant_i8(const uint8_t *q4, const uint8_t *s1, const uint8_t *z,
                       int64_t N, int64_t K, int8_t *r)
{
    int64_t G = K / ORC_GROUP, bad = 0;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t s = s1[n * G + k / ORC_GROUP];
            int64_t zz = z[n * G + k / ORC_GROUP];
            int64_t prod = (int64_t)q4[n * K + k] * s;
            int64_t zs = zz * s;
            int64_t v = prod - zs;
            if (v < -127 || v > 127 || prod > 240 || zs > 240)
                bad++;
            r[n * K + k] = (int8_t)clampi(v, -128, 127);
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Exact integer contraction: acc[m,n] = sum_k qx[m,k] * r[n,k] in int64,   */
/* stored as int32 (the main loop runs on INT8 matrix units with an INT32   */
/* accumulator: QServe talk summary, "Quantized Matrix Multiplication       */
/* (GEMM) Kernel on GPUs").  Returns the number of sums outside int32.      */
/* ------------------------------------------------------------------------ */
int64_t orc_gemm_acc(const int8_t *qx, const int8_t *r, int64_t M, int64_t N,
                     int64_t K, int32_t *acc)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; k++)
                sum += (int64_t)qx[m * K + k] * (int64_t)r[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN)
                bad++;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Epilogue: y = fp16( (float(acc) * s_a[m]) * float(s0[n]) ), fp32, in    */
/* that order (per-channel and per-token scales applied after the main      */
/* loop: QServe talk summary, "Progressive Group Quantization for W4A8      */
/* GEMM" and "Quantized Matrix Multiplication (GEMM) Kernel on GPUs").      */
/* ------------------------------------------------------------------------ */
void orc_epilogue(const int32_t *acc, const float *s_a, const uint16_t *s0,
                  int64_t M, int64_t N, uint16_t *y)
{
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            float t = (float)acc[m * N + n];
            t = t * s_a[m];
            t = t * orc_f16_to_f32(s0[n]);
            y[m * N + n] = orc_f32_to_f16(t);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* W4A16 on the same weights: fp16 activations times the dequantized        */
/* weights, no activation quantization.  QFactory notes 2.1 give the        */
/* dequantization w = (w_quant - zero) * scale with a half-precision scale; */
/* Lecture 15 notes 15.5 describe this int4 -> fp16 path inside the main    */
/* loop.  With this build's two-level weights the dequantized weight is     */
/* r[n,k] * s0[n], r = q4*s1 - z*s1 from orc_dequant_i8, so                 */
/*   ref[m,n]    = sum_k x[m,k] * r[n,k] * s0[n]     (double)               */
/*   absref[m,n] = sum_k |x[m,k] * r[n,k] * s0[n]|                          */
/* Each product is exact in double (11 + 7 + 11 significant bits); the sums */
/* are rounded, k in order.  absref scales the rounding error of an fp32    */
/* evaluation, for the tolerance of the comparison.                         */
/* ------------------------------------------------------------------------ */
void orc_gemm_w4a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *r,
                    const uint16_t *s0, int64_t N, double *ref, double *absref)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const double sc = (double)orc_f16_to_f32(s0[n]);
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, asum = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const double p = (double)orc_f16_to_f32(x[m * K + k]) * (double)r[n * K + k] * sc;
                sum = sum + p;
                asum = asum + fabs(p);
            }
            ref[m * N + n] = sum;
            absref[m * N + n] = asum;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* KV cache: 4-bit asymmetric quantization per (token, head).               */
/* The QServe talk summary ("Smooth Attention for K4V4 KV Cache             */
/* Compression", "Attention Computation Acceleration") stores keys and      */
/* values in 4 bits with zero points and scaling factors that the attention */
/* kernel prefetches, and ("Long Context Challenges") has those factors     */
/* grow with the sequence: one (scale, zero) per cached token and head.    */
/* The form is the QFactory notes' (2.1) asymmetric one,                    */
/*   x ~ (code - zero) * scale.                                             */
/* Readings, the same as the weights' level 2 where they apply:             */
/*   - the range includes 0: lo = min(0, min x), hi = max(0, max x), so the  */
/*     zero point lies in [0, 15] and 0 is represented exactly;            */
/*   - scale = fp16((hi - lo) / 15) (fp32 subtraction and IEEE division,    */
/*     then round to nearest even); the codes divide by that stored value;  */
/*   - zero = rint(-lo / scale) and code = rint(x / scale) + zero, both in  */
/*     fp32 with ties to even and clamped to [0, 15];                        */
/*   - a row whose scale rounds to 0 stores scale 0, zero 0 and codes 0.    */
/* x: fp16 bits [rows, D]; codes one per byte [rows, D]; s fp16 bits, z.    */
/* ------------------------------------------------------------------------ */
void orc_quantize_kv4(const uint16_t *x, int64_t rows, int64_t D, uint8_t *codes,
                      uint16_t *s, uint8_t *z)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; i++) {
        const uint16_t *xi = x + i * D;
        float lo = 0.0f, hi = 0.0f;
        for (int64_t d = 0; d < D; d++) {
            const float v = orc_f16_to_f32(xi[d]);
            if (v < lo)
                lo = v;
            if (v > hi)
                hi = v;
        }
        const uint16_t sh = orc_f32_to_f16((hi - lo) / 15.0f);
        const float sf = orc_f16_to_f32(sh);
        s[i] = sh;
        if (sf == 0.0f) {
            s[i] = 0;
            z[i] = 0;
            for (int64_t d = 0; d < D; d++)
                codes[i * D + d] = 0;
            continue;
        }
        const float zf = clampf(rintf(-lo / sf), 0.0f, 15.0f);
        z[i] = (uint8_t)zf;
        for (int64_t d = 0; d < D; d++) {
            const float t = rintf(orc_f16_to_f32(xi[d]) / sf) + zf;
            codes[i * D + d] = (uint8_t)clampf(t, 0.0f, 15.0f);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the 4-bit cache.  One new query token per          */
/* sequence; the cache is dequantized as (code - zero) * scale (QServe talk */
/* summary, "Attention Computation Acceleration": the 4-bit elements are    */
/* converted for the score computation; Lecture 15 notes, 15.6: the kernel  */
/* works on the int4 cache directly and never writes it back at higher      */
/* precision).  For sequence b and query head h, with kv head g = h / (Hq / */
/* Hkv) (consecutive query heads share a kv head) and L = lens[b] tokens:  */
/*   score_t = sm_scale * sum_d q[d] * kdq[t, d]          (t < L)           */
/*   p_t     = exp(score_t - max_t score_t)                                 */
/*   out[d]  = sum_t p_t vdq[t, d] / sum_t p_t                              */
/* all in double (each q * (code - zero) is exact, and the sums of those    */
/* exact products over D = 128 are exact too); L = 0 gives out = 0.         */
/* Also returned, for error bounds: absout[d] = sum_t p_t |vdq[t, d]| /     */
/* sum_t p_t, score_t and absscore_t = sm_scale * sum_d |q[d] kdq[t, d]|    */
/* (both 0 for t >= L).  Codes one per byte [B, Hkv, S, D]; scales fp16     */
/* bits and zeros [B, Hkv, S]; q [B, Hq, D] fp16 bits; out [B, Hq, D].      */
/* ------------------------------------------------------------------------ */
void orc_kv4_attention(const uint16_t *q, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                       const uint8_t *kc, const uint16_t *ks, const uint8_t *kz,
                       const uint8_t *vc, const uint16_t *vs, const uint8_t *vz,
                       int64_t S, const int32_t *lens, double sm_scale,
                       double *out, double *absout, double *score, double *absscore)
{
    const int64_t G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; b++) {
        for (int64_t h = 0; h < Hq; h++) {
            const int64_t g = h / G;
            const int64_t L = lens[b];
            const uint16_t *qh = q + (b * Hq + h) * D;
            const int64_t row0 = (b * Hkv + g) * S;      /* first cache row of (b, g) */
            double *sc = score + (b * Hq + h) * S;
            double *asc = absscore + (b * Hq + h) * S;
            double *o = out + (b * Hq + h) * D;
            double *ao = absout + (b * Hq + h) * D;
            for (int64_t t = 0; t < S; t++) {
                sc[t] = 0.0;
                asc[t] = 0.0;
            }
            for (int64_t d = 0; d < D; d++) {
                o[d] = 0.0;
                ao[d] = 0.0;
            }
            if (L == 0)
                continue;
            double mx = -INFINITY;
            for (int64_t t = 0; t < L; t++) {
                const double kscale = (double)orc_f16_to_f32(ks[row0 + t]);
                double dot = 0.0, adot = 0.0;
                for (int64_t d = 0; d < D; d++) {
                    const double kd = ((double)kc[(row0 + t) * D + d] - (double)kz[row0 + t]) * kscale;
                    const double prod = (double)orc_f16_to_f32(qh[d]) * kd;
                    dot = dot + prod;
                    adot = adot + fabs(prod);
                }
                sc[t] = sm_scale * dot;
                asc[t] = sm_scale * adot;
                if (sc[t] > mx)
                    mx = sc[t];
            }
            double den = 0.0;
            for (int64_t t = 0; t < L; t++)
                den = den + exp(sc[t] - mx);
            for (int64_t t = 0; t < L; t++) {
                const double p = exp(sc[t] - mx);
                const double vscale = (double)orc_f16_to_f32(vs[row0 + t]);
                for (int64_t d = 0; d < D; d++) {
                    const double vd = ((double)vc[(row0 + t) * D + d] - (double)vz[row0 + t]) * vscale;
                    o[d] = o[d] + p * vd;
                    ao[d] = ao[d] + p * fabs(vd);
                }
            }
            for (int64_t d = 0; d < D; d++) {
                o[d] = o[d] / den;
                ao[d] = ao[d] / den;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The whole serving-time path for one call, from fp16 activations and the  */
/* level-2 weight form to fp16 outputs.  Used to time the oracle.           */
/* r (int8 [N,K]) is caller-provided scratch.  Returns the number of        */
/* threads used by the contraction.                                         */
/* ------------------------------------------------------------------------ */
int orc_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *q4,
               const uint8_t *s1, const uint8_t *z, const uint16_t *s0,
               int64_t N, int8_t *qx, float *s_a, int8_t *r, int32_t *acc,
               uint16_t *y)
{
    orc_quantize_act(x, M, K, K, qx, s_a);
    orc_dequant_i8(q4, s1, z, N, K, r);
    orc_gemm_acc(qx, r, M, N, K, acc);
    orc_epilogue(acc, s_a, s0, M, N, y);
    return orc_num_threads();
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
