/*
 * afq_oracle.c -- CPU reference for fused activation FP8 quantisation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle the GPU kernels are
 * checked against.  Only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg load it; the product path never does.  It shares no code,
 * table or constant generator with the HIP kernels.
 *
 * It is deliberately plain and slow:
 *   - every number format is decoded from its field definition, and rounding
 *     to a format means "pick the nearest representable value, ties to the
 *     even code", found by searching the sorted table of decoded values;
 *   - the normalisation arithmetic is carried out in fp64 and rounded once
 *     to the activation dtype;
 *   - the fused operations are computed as the unfused composition
 *     (norm, then round to the activation dtype, then quantise), because the
 *     fused kernels are specified as reaching that same result.
 * The only places where fp32 is used on purpose are where the pages fix it:
 * the fp32 group/token scale amax/448 and the fp32 quotient u/s that is
 * rounded to e4m3, the fp32 SiLU-and-mul activation of the MXFP8 path, and
 * the fp32 normed value of the fp32-direct norm variant.
 *
 * Sources (the pages):
 *   [P1] vLLM pull request 65478, "MiniMax-M3.1: fuse the FFN-side MXFP8
 *        activation quant into the post-attention add+RMSNorm and swiglu".
 *   [P2] SGLang pull request 48043, "[Perf] [AMD] qwen3: Fuse the 1x128 FP8
 *        input quant into RMSNorm and SiLU-and-mul for block-FP8 linears on
 *        gfx950".
 *   [P3] vLLM pull request 65479, "AiterMxfp8LinearKernel" (MXFP8 consumer).
 *   [P4] SGLang pull request 34502, "[ROCm] Fuse per-token activation quant
 *        into RMSNorm for per-channel quantized attention".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Constants of the interface (mirrored, not shared, by the Python wrapper). */
enum { ORC_MXFP8 = 0, ORC_BLOCK128 = 1, ORC_PER_TOKEN = 2 };
enum { ORC_BF16 = 0, ORC_FP16 = 1, ORC_FP32 = 2 };
enum { ORC_RMSNORM_STANDARD = 0, ORC_RMSNORM_GEMMA = 1 };
/* What the quantiser is applied to: the default of each path, the fp32
 * normed value (norm), or the bf16-rounded fp32 activation (MXFP8 SiLU). */
enum { ORC_QIN_DEFAULT = 0, ORC_QIN_FP32 = 1, ORC_QIN_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats, decoded from their field definitions.                     */
/* Each takes a non-negative code (sign bit clear) and returns its value.    */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
static double dec_bf16(uint32_t c)
{
    uint32_t e = (c >> 7) & 0xFFu, m = c & 0x7Fu;
    if (e == 0) return ldexp((double)m, -126 - 7);          /* subnormal */
    return ldexp(1.0 + (double)m / 128.0, (int)e - 127);
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
static double dec_fp16(uint32_t c)
{
    uint32_t e = (c >> 10) & 0x1Fu, m = c & 0x3FFu;
    if (e == 0) return ldexp((double)m, -14 - 10);
    return ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, so the largest finite magnitude is
 * S.1111.110 = 1.75 * 2^8 = 448.  Subnormals are m * 2^-9. */
static double dec_e4m3(uint32_t c)
{
    uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
    if (e == 0) return ldexp((double)m, -6 - 3);
    return ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

/* Sorted tables of the non-negative finite values (index == code). */
#define N_BF16 0x7F80u /* codes 0x0000..0x7F7F; 0x7F80 is +inf */
#define N_FP16 0x7C00u /* codes 0x0000..0x7BFF; 0x7C00 is +inf */
#define N_E4M3 0x7Fu   /* codes 0x00..0x7E;     0x7F is NaN    */
static double tab_bf16[N_BF16], tab_fp16[N_FP16], tab_e4m3[N_E4M3];
static pthread_once_t tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (uint32_t c = 0; c < N_BF16; ++c) tab_bf16[c] = dec_bf16(c);
    for (uint32_t c = 0; c < N_FP16; ++c) tab_fp16[c] = dec_fp16(c);
    for (uint32_t c = 0; c < N_E4M3; ++c) tab_e4m3[c] = dec_e4m3(c);
}
static void tables(void) { pthread_once(&tab_once, build_tables); }

/*
 * Round a magnitude a + tail to the nearest entry of a sorted value table,
 * ties to the even code.  a is an fp64 value and tail a much smaller
 * correction (zero for a plain fp64 input) that only matters when a sits
 * exactly on the midpoint of two table values.  `beyond` is the value the
 * format's exponent range would give the code after the largest finite one
 * (2^128 for bf16, 2^16 for fp16): a magnitude at or past the midpoint
 * between the largest finite value and `beyond` overflows and the function
 * returns n (the infinity code).  Every comparison is exact: the midpoint
 * of two adjacent table values is representable in fp64.
 */
static uint32_t nearest_code(const double *tab, uint32_t n, double beyond, double a, double tail)
{
    uint32_t lo, hi;
    if (a >= tab[n - 1]) {
        lo = n - 1;
        hi = n;
    } else {
        /* largest lo with tab[lo] <= a */
        lo = 0;
        hi = n - 1;
        while (hi - lo > 1) {
            uint32_t mid = lo + (hi - lo) / 2;
            if (tab[mid] <= a) lo = mid; else hi = mid;
        }
        hi = lo + 1;
    }
    double upper = hi < n ? tab[hi] : beyond;
    double mid = (tab[lo] + upper) / 2.0;
    if (a < mid) return lo;
    if (a > mid) return hi;
    if (tail > 0.0) return hi;
    if (tail < 0.0) return lo;
    return (lo & 1u) ? hi : lo;
}

/* Round a real value to bf16 / fp16, round-to-nearest-even.  Returns the
 * 16-bit code.  The input may be any fp64 value; it is rounded once. */
uint16_t orc_round_bf16(double v)
{
    tables();
    uint32_t s = signbit(v) ? 0x8000u : 0u;
    return (uint16_t)(s | nearest_code(tab_bf16, N_BF16, ldexp(1.0, 128), fabs(v), 0.0));
}

/* Round the two-term value hi + lo (|lo| below half an fp64 ulp of hi) to
 * bf16: the tail decides only an exact midpoint of hi. */
static uint16_t round_bf16_2(double hi, double lo)
{
    tables();
    uint32_t s = signbit(hi) ? 0x8000u : 0u;
    return (uint16_t)(s | nearest_code(tab_bf16, N_BF16, ldexp(1.0, 128), fabs(hi),
                                       signbit(hi) ? -lo : lo));
}

/* Round hi + lo to fp32 (nearest even), the tail deciding an exact tie. */
static float round_f32_2(double hi, double lo)
{
    float f = (float)hi;
    if ((double)f == hi) return f;
    /* hi lies strictly between two adjacent fp32 values */
    float below = (double)f < hi ? f : nextafterf(f, -INFINITY);
    float above = (double)f > hi ? f : nextafterf(f, INFINITY);
    double mid = ((double)below + (double)above) / 2.0;
    if (hi != mid) return f;
    if (lo > 0.0) return above;
    if (lo < 0.0) return below;
    return f; /* RNE already picked the even neighbour */
}

uint16_t orc_round_fp16(double v)
{
    tables();
    uint32_t s = signbit(v) ? 0x8000u : 0u;
    return (uint16_t)(s | nearest_code(tab_fp16, N_FP16, ldexp(1.0, 16), fabs(v), 0.0));
}

/* Round to OCP e4m3fn, round-to-nearest-even.  The caller has clamped the
 * value to [-448, 448] (the saturating rule of the quantiser); the sign goes
 * to bit 7, so -0 and negative values that round to zero give 0x80. */
uint8_t orc_round_e4m3(double v)
{
    tables();
    double a = fabs(v);
    if (a > 448.0) a = 448.0; /* defensive; callers clamp first */
    uint32_t s = signbit(v) ? 0x80u : 0u;
    return (uint8_t)(s | nearest_code(tab_e4m3, N_E4M3, 512.0, a, 0.0));
}

double orc_decode_bf16(uint16_t c) { double v = dec_bf16(c & 0x7FFFu); return (c & 0x8000u) ? -v : v; }
double orc_decode_fp16(uint16_t c) { double v = dec_fp16(c & 0x7FFFu); return (c & 0x8000u) ? -v : v; }
double orc_decode_e4m3(uint8_t c)  { double v = dec_e4m3(c & 0x7Fu);   return (c & 0x80u) ? -v : v; }

/* ------------------------------------------------------------------------ */
/* Quantisation of one row of activation values u[0..n) (each exactly a     */
/* value of the quantised dtype: bf16, fp16 or fp32).                       */

/*
 * E8M0 scale byte of an MXFP8 block (OCP Microscaling Formats v1.0, the
 * shared-scale rule used for MXFP8 activations in [P1] and consumed
 * row-major by the GEMMs of [P1] "Limitations" and [P3]).  The shared
 * exponent is floor(log2(amax)) minus the largest exponent of e4m3 (8);
 * for an fp32 amax floor(log2) is read from the biased exponent field E.
 * The byte is E - 8, clamped below at 0 (2^-127) for zero, subnormal and
 * tiny blocks.
 */
uint8_t orc_e8m0_byte(float amax)
{
    uint32_t bits;
    memcpy(&bits, &amax, 4);
    int E = (int)((bits >> 23) & 0xFFu);
    int b = E - 8;
    return (uint8_t)(b > 0 ? b : 0);
}

static double clamp448(double v)
{
    if (v > 448.0) return 448.0;
    if (v < -448.0) return -448.0;
    return v;
}

/* MXFP8: groups of 32, E8M0 scale X = 2^(b-127), codes e4m3(clamp(u/X)). */
static void quant_mx_group(const double *u, int g, uint8_t *q, uint8_t *sbyte)
{
    double amax = 0.0;
    for (int j = 0; j < g; ++j) if (fabs(u[j]) > amax) amax = fabs(u[j]);
    uint8_t b = orc_e8m0_byte((float)amax); /* amax is a dtype value: exact in fp32 */
    *sbyte = b;
    for (int j = 0; j < g; ++j) {
        double v = ldexp(u[j], 127 - (int)b); /* u / X, exact */
        q[j] = orc_round_e4m3(clamp448(v));
    }
}

/* Block (1x128) and per-token: fp32 scale s = amax / 448 ([P2]
 * "Modifications": the per-1x128 quant; [P4] "Change": x_scale[m,1]); the
 * code is e4m3 of the fp32 quotient u/s, clamped to +-448.  A group whose
 * stored scale is 0 -- all zero, or an amax so small (at most 224 * 2^-149)
 * that amax / 448 underflows fp32 -- has codes 0x00: with s = 0 every
 * dequantised value is 0, as for the all-zero group. */
static void quant_fp32scale_group(const double *u, int g, uint8_t *q, float *s_out)
{
    double amax = 0.0;
    for (int j = 0; j < g; ++j) if (fabs(u[j]) > amax) amax = fabs(u[j]);
    float A = (float)amax;
    float s = A / 448.0f; /* IEEE fp32 division */
    *s_out = s;
    for (int j = 0; j < g; ++j) {
        if (s == 0.0f) { q[j] = 0x00; continue; }
        float t = (float)u[j] / s; /* IEEE fp32 division */
        q[j] = orc_round_e4m3(clamp448((double)t));
    }
}

/* Quantise one row.  MX scales are bytes, block/per-token scales fp32. */
static void quant_row(const double *u, int64_t n, int mode, uint8_t *q, void *scales)
{
    if (mode == ORC_MXFP8) {
        for (int64_t k = 0; k < n / 32; ++k)
            quant_mx_group(u + 32 * k, 32, q + 32 * k, (uint8_t *)scales + k);
    } else if (mode == ORC_BLOCK128) {
        for (int64_t k = 0; k < n / 128; ++k)
            quant_fp32scale_group(u + 128 * k, 128, q + 128 * k, (float *)scales + k);
    } else {
        quant_fp32scale_group(u, (int)n, q, (float *)scales);
    }
}

static int64_t scales_per_row(int64_t n, int mode)
{
    return mode == ORC_MXFP8 ? n / 32 : mode == ORC_BLOCK128 ? n / 128 : 1;
}
static int64_t scale_bytes(int mode) { return mode == ORC_MXFP8 ? 1 : 4; }

static double load_dt(const void *p, int64_t i, int dtype)
{
    if (dtype == ORC_BF16) return orc_decode_bf16(((const uint16_t *)p)[i]);
    if (dtype == ORC_FP16) return orc_decode_fp16(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

static uint16_t round_dt(double v, int dtype)
{
    return dtype == ORC_FP16 ? orc_round_fp16(v) : orc_round_bf16(v);
}

static double decode_dt16(uint16_t c, int dtype)
{
    return dtype == ORC_FP16 ? orc_decode_fp16(c) : orc_decode_bf16(c);
}

/* ------------------------------------------------------------------------ */
/* Standalone row-wise quantisation of an activation [M, n] (the "separate  */
/* quant" that the fused kernels replace: [P1] mxfp8_e4m3_quantize, [P2]    */
/* per-1x128 quant, [P4] standalone per-token quant).  Rows [r0, r1).        */
int orc_quant_rows(int64_t M, int64_t n, const void *x, int64_t x_stride, int in_dtype,
                   int mode, uint8_t *values, void *scales, int64_t r0, int64_t r1,
                   double *work /* n doubles */)
{
    (void)M;
    int64_t spr = scales_per_row(n, mode), sb = scale_bytes(mode);
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < n; ++j) work[j] = load_dt(x, i * x_stride + j, in_dtype);
        quant_row(work, n, mode, values + i * n, (uint8_t *)scales + i * spr * sb);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/*
 * (residual add +) RMSNorm + quantisation, rows [r0, r1) of one segment.
 *
 *   h_j   = RNE_dt(x_j + r_j)            residual add; h is written back
 *                                        ([P1] microbench: residual output
 *                                        compared bitwise with the unfused op)
 *   ms    = (sum_j h_j^2) / H            mean over the H columns
 *   inv   = 1 / sqrt(ms + eps)
 *   y_j   = h_j * inv * g_j              g_j = 1 + w_j (Gemma), w_j (standard)
 *   u_j   = RNE_dt(y_j)                  the normed row as the unfused norm
 *                                        stores it; also the optional copy
 *   (q, s) = quant(u)                    [P1] "Test Plan / Correctness": the
 *                                        fused output equals norm followed by
 *                                        mxfp8_e4m3_quantize; the same
 *                                        composition is taken for the 1x128
 *                                        ([P2]) and per-token ([P4]) modes.
 *
 * ms, inv and y are evaluated in fp64 and rounded once to the dtype.
 *
 * qin = ORC_QIN_FP32, the fp32-direct variant ([P2] "Accuracy Tests": the
 * AITER fused 1x128 norm quantises the fp32 normalized value itself, where
 * the unfused chain first rounds it to bf16).  The pages do not give its
 * fp32 arithmetic; it is taken in the plain order, every step rounded to
 * fp32 once:
 *   inv32 = fl32(1 / sqrt(ms + eps))     ms as above (fp64)
 *   g32_j = fl32(1 + w_j) (Gemma), w_j (standard)
 *   y_j   = fl32(fl32(h_j * inv32) * g32_j)
 *   normed_j = RNE_dt(y_j);  (q, s) = quant(y)
 *
 * residual / h_out may be NULL (plain RMSNorm: h = x).  normed may be NULL.
 */
int orc_norm_quant_rows(int64_t M, int64_t H, const void *x, int64_t x_stride,
                        const void *residual, void *h_out, const void *weight,
                        int kind, int dtype, int mode, int qin, float eps,
                        uint8_t *values, void *scales, void *normed,
                        int64_t r0, int64_t r1, double *work /* 2H doubles */)
{
    (void)M;
    double *h = work, *u = work + H;
    int64_t spr = scales_per_row(H, mode), sb = scale_bytes(mode);
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < H; ++j) {
            double xv = load_dt(x, i * x_stride + j, dtype);
            if (residual) {
                double rv = load_dt(residual, i * H + j, dtype);
                uint16_t hc = round_dt(xv + rv, dtype); /* exact sum, one rounding */
                if (h_out) ((uint16_t *)h_out)[i * H + j] = hc;
                h[j] = decode_dt16(hc, dtype);
            } else {
                h[j] = xv;
            }
        }
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) ss += h[j] * h[j];
        double ms = ss / (double)H;
        double inv = 1.0 / sqrt(ms + (double)eps);
        if (qin == ORC_QIN_FP32) {
            float inv32 = (float)inv;
            for (int64_t j = 0; j < H; ++j) {
                float w32 = (float)load_dt(weight, j, dtype); /* a dtype value: exact */
                float g32 = (kind == ORC_RMSNORM_GEMMA) ? 1.0f + w32 : w32;
                float t32 = (float)h[j] * inv32;
                float y32 = t32 * g32;
                if (normed) ((uint16_t *)normed)[i * H + j] = round_dt((double)y32, dtype);
                u[j] = (double)y32;
            }
        } else {
            for (int64_t j = 0; j < H; ++j) {
                double w = load_dt(weight, j, dtype);
                double g = (kind == ORC_RMSNORM_GEMMA) ? 1.0 + w : w;
                uint16_t uc = round_dt(h[j] * inv * g, dtype);
                if (normed) ((uint16_t *)normed)[i * H + j] = uc;
                u[j] = decode_dt16(uc, dtype);
            }
        }
        quant_row(u, H, mode, values + i * H, (uint8_t *)scales + i * spr * sb);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/*
 * SiLU.  silu(g) = g / (1 + e^-g) = g e^g / (1 + e^g), evaluated in fp64 as
 * a two-term value hi + lo.  For |g| < 1/2 it is written g/2 + (g/2)
 * tanh(g/2) (the same function, since the logistic function equals
 * (1 + tanh(g/2)) / 2): for tiny g the fp64 quotient collapses to exactly
 * g/2, which can be a bf16 or fp32 rounding midpoint, while the true value
 * lies beyond it by about g^2/4; the second term keeps that information.
 */
static void silu_2(double g, double *hi, double *lo)
{
    if (g == 0.0) { /* g * logistic(g) keeps the sign of a zero gate */
        *hi = g;
        *lo = 0.0;
        return;
    }
    if (fabs(g) < 0.5) {
        double a = g / 2.0, b = (g / 2.0) * tanh(g / 2.0);
        double s = a + b;           /* |a| >= |b|: the error of s is exact */
        *hi = s;
        *lo = b - (s - a);
        return;
    }
    if (g < 0.0) {
        double e = exp(g);
        *hi = g * e / (1.0 + e);
    } else {
        *hi = g / (1.0 + exp(-g));
    }
    *lo = 0.0;
}

double orc_silu(double g)
{
    double hi, lo;
    silu_2(g, &hi, &lo);
    return hi + lo;
}

/*
 * SiLU-and-mul + quantisation, rows [r0, r1).  The input row is
 * [gate | up], gate in columns [0, I), up in [I, 2I) ([P1] swiglu "split"
 * layout).
 *
 * MXFP8 ([P1] "Purpose", commit 2 and "Test Plan": the SiLU-and-mul is
 * evaluated in fp32 and its fp32 result goes straight into the quantiser,
 * with no bf16 rounding).  In fp32 arithmetic silu is an fp32 value before
 * it multiplies up, so:
 *     s_j = fl32(silu(g_j)),  a_j = fl32(s_j * u_j)
 *     scale from the fp32 block amax, codes e4m3(clamp(a_j / X)).
 * (For g below about -87, silu(g) is an fp32 subnormal or zero, and so is
 * a_j unless |u_j| is large.)
 * BLOCK128 ([P2] "Modifications": the fused kernel takes the same two bf16
 * roundings as the unfused SiLU-and-mul, silu first and then the product,
 * so its output equals the unfused path):
 *     a_j = RNE_bf16(RNE_bf16(silu(g_j)) * u_j), then the 1x128 quant.
 * The pages pair SiLU-and-mul with no per-token quant; that mode is rejected
 * (returns -1).  act_out (optional) receives RNE_bf16(a_j).
 *
 * qin = ORC_QIN_BF16 with MXFP8, the bf16-first variant: the quantiser
 * reads RNE_bf16(a_j), the activation as the unfused chain stores it before
 * its separate quant ([P1] "Test Plan / Correctness" and the review: the
 * fused kernel skips that bf16 rounding, the unfused chain takes it).
 */
int orc_silu_quant_rows(int64_t M, int64_t I, const uint16_t *gu, int64_t gu_stride,
                        int mode, int qin, uint8_t *values, void *scales, uint16_t *act_out,
                        int64_t r0, int64_t r1, double *work /* I doubles */)
{
    (void)M;
    if (mode != ORC_MXFP8 && mode != ORC_BLOCK128) return -1;
    int64_t spr = scales_per_row(I, mode), sb = scale_bytes(mode);
    for (int64_t i = r0; i < r1; ++i) {
        const uint16_t *row = gu + i * gu_stride;
        for (int64_t j = 0; j < I; ++j) {
            double g = orc_decode_bf16(row[j]);
            double u = orc_decode_bf16(row[I + j]);
            double shi, slo, a;
            silu_2(g, &shi, &slo);
            if (mode == ORC_MXFP8) {
                /* s = fl32(silu(g)) from the two-term value; s * u of a
                 * 24-bit and an 8-bit significand is exact in fp64, so one
                 * more rounding gives fl32(s * u) */
                double s32 = (double)round_f32_2(shi, slo);
                a = (double)round_f32_2(s32 * u, 0.0);
            } else {
                double sg = orc_decode_bf16(round_bf16_2(shi, slo));
                a = orc_decode_bf16(orc_round_bf16(sg * u)); /* sg*u exact in fp64 */
            }
            uint16_t ac = orc_round_bf16(a);
            if (mode == ORC_MXFP8 && qin == ORC_QIN_BF16) a = orc_decode_bf16(ac);
            work[j] = a;
            if (act_out) act_out[i * I + j] = ac;
        }
        quant_row(work, I, mode, values + i * I, (uint8_t *)scales + i * spr * sb);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/*
 * Clamped SwiGLU ("swiglu_oai" in [P1]'s benchmark script, called there with
 * alpha = 1.702, beta = 1.0, limit = 7.0 on the split [gate | up] layout).
 * The pages name the function and its three parameters but do not write it
 * out; the reading taken is the clamped SwiGLU published with OpenAI's
 * gpt-oss models, per element:
 *     gc  = min(g, limit)                    (gate clamped from above only)
 *     uc  = min(max(u, -limit), limit)       (up clamped on both sides)
 *     glu = gc * logistic(alpha * gc)
 *     a   = glu * (uc + beta)
 * MXFP8, fp32 arithmetic as in the SiLU path ([P1] "Purpose", commit 2: the
 * swiglu is evaluated in fp32 and quantised in the same pass): each of glu,
 * uc + beta and their product is rounded to fp32 once,
 *     a_j = fl32(fl32(glu_j) * fl32(uc_j + beta)),
 * with alpha, beta and limit taken as the fp32 values the caller passes.
 * qin = ORC_QIN_BF16: the quantiser reads RNE_bf16(a_j), the activation as
 * the unfused swiglu -> quant chain stores it ([P1] "Test Plan /
 * Correctness").  act_out (optional) receives RNE_bf16(a_j).  Only MXFP8
 * (returns -1 otherwise).
 */

/* glu = gc * logistic(z), z = alpha * gc, as a two-term value hi + lo.  For
 * |z| < 1/2 it is written gc/2 + (gc/2) tanh(z/2) (logistic(z) = (1 +
 * tanh(z/2)) / 2), so that for tiny gates the information beyond gc/2 is
 * kept in the second term; otherwise gc e^z / (1 + e^z) (z < 0, no
 * overflow) or gc / (1 + e^-z).  A zero gate keeps its sign. */
static void glu_2(double gc, double z, double *hi, double *lo)
{
    *lo = 0.0;
    if (gc == 0.0) {
        *hi = gc;
        return;
    }
    if (fabs(z) < 0.5) {
        double a = gc / 2.0, b = (gc / 2.0) * tanh(z / 2.0);
        double s = a + b;
        *hi = s;
        *lo = b - (s - a);   /* |a| >= |b|: exact error of the sum */
        return;
    }
    if (z < 0.0) {
        double e = exp(z);
        *hi = gc * e / (1.0 + e);
    } else {
        *hi = gc / (1.0 + exp(-z));
    }
}

/* fl32(glu) of a gate: gc = min(g, limit), alpha * gc exact in fp64 (a
 * 24-bit times an at most 24-bit significand) */
float orc_swiglu_glu32(double g, float alpha, float limit)
{
    double gc = g < (double)limit ? g : (double)limit;
    double hi, lo;
    glu_2(gc, (double)alpha * gc, &hi, &lo);
    return round_f32_2(hi, lo);
}

/* The fp32 activation a = fl32(fl32(glu) * fl32(uc + beta)). */
float orc_swiglu_act32(double g, double u, float alpha, float beta, float limit)
{
    double L = (double)limit, B = (double)beta;
    double uc = u < -L ? -L : (u > L ? L : u);
    double glu32 = (double)orc_swiglu_glu32(g, alpha, limit);
    /* uc + beta with its exact error (two-sum), rounded once */
    double s = uc + B, bb = s - uc;
    double err = (uc - (s - bb)) + (B - bb);
    double lin32 = (double)round_f32_2(s, err);
    /* the product of two fp32 values is exact in fp64 */
    return round_f32_2(glu32 * lin32, 0.0);
}

int orc_swiglu_oai_quant_rows(int64_t M, int64_t I, const uint16_t *gu, int64_t gu_stride,
                              int mode, int qin, float alpha, float beta, float limit,
                              uint8_t *values, void *scales, uint16_t *act_out,
                              int64_t r0, int64_t r1, double *work /* I doubles */)
{
    (void)M;
    if (mode != ORC_MXFP8) return -1;
    int64_t spr = scales_per_row(I, mode), sb = scale_bytes(mode);
    for (int64_t i = r0; i < r1; ++i) {
        const uint16_t *row = gu + i * gu_stride;
        for (int64_t j = 0; j < I; ++j) {
            double a = (double)orc_swiglu_act32(orc_decode_bf16(row[j]), orc_decode_bf16(row[I + j]),
                                                alpha, beta, limit);
            uint16_t ac = orc_round_bf16(a);
            if (qin == ORC_QIN_BF16) a = orc_decode_bf16(ac);
            work[j] = a;
            if (act_out) act_out[i * I + j] = ac;
        }
        quant_row(work, I, mode, values + i * I, (uint8_t *)scales + i * spr * sb);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the tests (element-wise application of the above).     */
void orc_round_bf16_n(const double *v, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(v[i]); }
void orc_round_fp16_n(const double *v, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_round_fp16(v[i]); }
void orc_round_e4m3_n(const double *v, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_round_e4m3(v[i]); }
void orc_e8m0_byte_n(const float *a, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_byte(a[i]); }
void orc_silu_n(const double *g, double *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_silu(g[i]); }
void orc_swiglu_glu32_n(const double *g, float *out, int64_t n, float alpha, float limit)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_swiglu_glu32(g[i], alpha, limit); }
void orc_swiglu_act32_n(const double *g, const double *u, float *out, int64_t n, float alpha,
                        float beta, float limit)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_swiglu_act32(g[i], u[i], alpha, beta, limit); }
