/*
 * afq_c_example.c -- the library used from plain C, with no Python or torch.
 *
 * Allocates device buffers with hipMalloc, calls the three entry points of
 * include/afq.h on seeded inputs, copies the outputs back and checks them
 * against the CPU oracle (oracle/afq_oracle.c, linked into this test
 * program): the fused add + Gemma RMSNorm + MXFP8 + copy, the 1x128
 * SiLU-and-mul, the clamped SwiGLU + MXFP8 and the standalone per-token
 * quantiser; and that the unfused chain (a copy-only norm launch, then
 * fp8_quant) reproduces the fused launch bit for bit.  Also checks the
 * version and an error path.  Prints one line per check; exits non-zero on
 * the first failure.
 */
#include "afq.h"

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's row functions (C linkage) */
int orc_norm_quant_rows(int64_t M, int64_t H, const void *x, int64_t x_stride,
                        const void *residual, void *h_out, const void *weight,
                        int kind, int dtype, int mode, int qin, float eps,
                        uint8_t *values, void *scales, void *normed,
                        int64_t r0, int64_t r1, double *work);
int orc_silu_quant_rows(int64_t M, int64_t I, const uint16_t *gu, int64_t gu_stride,
                        int mode, int qin, uint8_t *values, void *scales, uint16_t *act_out,
                        int64_t r0, int64_t r1, double *work);
int orc_swiglu_oai_quant_rows(int64_t M, int64_t I, const uint16_t *gu, int64_t gu_stride,
                              int mode, int qin, float alpha, float beta, float limit,
                              uint8_t *values, void *scales, uint16_t *act_out,
                              int64_t r0, int64_t r1, double *work);
int orc_quant_rows(int64_t M, int64_t n, const void *x, int64_t x_stride, int in_dtype,
                   int mode, uint8_t *values, void *scales, int64_t r0, int64_t r1, double *work);

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); exit(2); } } while (0)
#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); exit(1); } while (0)

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* xorshift64*, in (0, 1) */
{
    rs ^= rs >> 12; rs ^= rs << 25; rs ^= rs >> 27;
    return ((rs * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0) + 1e-300;
}
static double normal(void) { return sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform()); }

static uint16_t to_bf16(float f) /* round to nearest even (finite inputs) */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *dmalloc(size_t n) { void *p; CHECK_HIP(hipMalloc(&p, n)); return p; }
static void up(void *d, const void *h, size_t n) { CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice)); }
static void down(void *h, const void *d, size_t n) { CHECK_HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost)); }

/* monotone integer orders of the encodings */
static int ord16(uint16_t b) { return (b & 0x8000) ? -(int)(b & 0x7FFF) : (int)(b & 0x7FFF); }
static int ord8(uint8_t b) { return (b & 0x80) ? -(int)(b & 0x7F) : (int)(b & 0x7F); }

/* the agreement required of the library: 16-bit outputs <= 1 ulp, codes
 * equal or one step apart in <= 0.1 % (at least one), scales exact in all
 * but 0.1 % */
static void compare16(const char *what, const uint16_t *a, const uint16_t *b, size_t n, int exact)
{
    size_t off = 0;
    for (size_t i = 0; i < n; ++i) {
        int d = abs(ord16(a[i]) - ord16(b[i]));
        if (d > (exact ? 0 : 1)) FAIL("%s: element %zu differs by %d", what, i, d);
        off += d != 0;
    }
    printf("%s: %zu elements, %zu one ulp apart\n", what, n, off);
}
static void compare_codes(const char *what, const uint8_t *a, const uint8_t *b, size_t n)
{
    size_t one = 0, budget = n / 1000 > 0 ? n / 1000 : 1;
    for (size_t i = 0; i < n; ++i) {
        int d = abs(ord8(a[i]) - ord8(b[i]));
        if (d > 1) FAIL("%s: code %zu differs by %d", what, i, d);
        one += d == 1;
    }
    if (one > budget) FAIL("%s: %zu codes one step apart", what, one);
    printf("%s: %zu codes, %zu one step apart\n", what, n, one);
}
static void compare_bytes(const char *what, const void *a, const void *b, size_t n, size_t elt)
{
    size_t bad = 0, groups = n / elt, budget = groups / 1000 > 0 ? groups / 1000 : 1;
    for (size_t g = 0; g < groups; ++g)
        bad += memcmp((const char *)a + g * elt, (const char *)b + g * elt, elt) != 0;
    if (bad > budget) FAIL("%s: %zu of %zu scales inexact", what, bad, groups);
    printf("%s: %zu scales, %zu inexact\n", what, groups, bad);
}

int main(void)
{
    if (afq_abi_version() != AFQ_ABI_VERSION) FAIL("ABI version %d, header %d", afq_abi_version(), AFQ_ABI_VERSION);
    if (fused_add_rmsnorm_quant(NULL, NULL) != AFQ_ERR_NULL) FAIL("NULL descriptor not rejected");
    printf("abi version %d; NULL descriptor -> %s\n", afq_abi_version(), afq_status_string(AFQ_ERR_NULL));

    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    double *work = malloc(sizeof(double) * 2 * 32768);

    /* ---- fused add + Gemma RMSNorm + MXFP8 + bf16 copy, M = 37, H = 6144 */
    {
        const int64_t M = 37, H = 6144;
        uint16_t *x = malloc(2 * M * H), *r = malloc(2 * M * H), *w = malloc(2 * H);
        for (int64_t i = 0; i < M * H; ++i) x[i] = to_bf16((float)(3.0 * normal()));
        for (int64_t i = 0; i < M * H; ++i) r[i] = to_bf16((float)normal());
        for (int64_t j = 0; j < H; ++j) w[j] = to_bf16((float)(0.1 * normal()));
        void *dx = dmalloc(2 * M * H), *dr = dmalloc(2 * M * H), *dw = dmalloc(2 * H);
        void *dh = dmalloc(2 * M * H), *dq = dmalloc(M * H), *ds = dmalloc(M * H / 32), *dn = dmalloc(2 * M * H);
        up(dx, x, 2 * M * H); up(dr, r, 2 * M * H); up(dw, w, 2 * H);
        afq_norm_desc d;
        memset(&d, 0, sizeof d);
        d.M = M; d.nseg = 1; d.kind = AFQ_RMSNORM_GEMMA; d.dtype = AFQ_BF16; d.mode = AFQ_MXFP8;
        d.eps = 1e-6f; d.quant_input = AFQ_QIN_DEFAULT;
        d.residual_in = dr; d.residual_out = dh;
        d.seg[0].x = dx; d.seg[0].x_row_stride = H; d.seg[0].weight = dw; d.seg[0].cols = H;
        d.seg[0].out.values = dq; d.seg[0].out.scales = ds; d.seg[0].out.normed = dn;
        int stt = fused_add_rmsnorm_quant(&d, st);
        if (stt != AFQ_OK) FAIL("fused_add_rmsnorm_quant: %s", afq_status_string(stt));
        CHECK_HIP(hipStreamSynchronize(st));
        uint16_t *gh = malloc(2 * M * H), *gn = malloc(2 * M * H), *oh = malloc(2 * M * H), *on = malloc(2 * M * H);
        uint8_t *gq = malloc(M * H), *gs = malloc(M * H / 32), *oq = malloc(M * H), *os = malloc(M * H / 32);
        down(gh, dh, 2 * M * H); down(gn, dn, 2 * M * H); down(gq, dq, M * H); down(gs, ds, M * H / 32);
        orc_norm_quant_rows(M, H, x, H, r, oh, w, 1, 0, 0, 0, 1e-6f, oq, os, on, 0, M, work);
        compare16("norm residual h", gh, oh, M * H, 1);
        compare16("norm bf16 copy", gn, on, M * H, 0);
        compare_codes("norm MXFP8 codes", gq, oq, M * H);
        compare_bytes("norm E8M0 scales", gs, os, M * H / 32, 1);

        /* the unfused chain: a copy-only norm launch (values and scales NULL),
         * then fp8_quant of its rows -- bit-identical to the fused launch */
        void *dh2 = dmalloc(2 * M * H), *dn2 = dmalloc(2 * M * H), *dq2 = dmalloc(M * H), *ds2 = dmalloc(M * H / 32);
        d.residual_out = dh2;
        d.seg[0].out.values = NULL; d.seg[0].out.scales = NULL; d.seg[0].out.normed = dn2;
        stt = fused_add_rmsnorm_quant(&d, st);
        if (stt != AFQ_OK) FAIL("copy-only fused_add_rmsnorm_quant: %s", afq_status_string(stt));
        afq_quant_desc qd;
        memset(&qd, 0, sizeof qd);
        qd.M = M; qd.cols = H; qd.x = dn2; qd.x_row_stride = H; qd.dtype = AFQ_BF16; qd.mode = AFQ_MXFP8;
        qd.out.values = dq2; qd.out.scales = ds2;
        stt = fp8_quant(&qd, st);
        if (stt != AFQ_OK) FAIL("fp8_quant of the copy-only rows: %s", afq_status_string(stt));
        CHECK_HIP(hipStreamSynchronize(st));
        uint16_t *ch = malloc(2 * M * H), *cn = malloc(2 * M * H);
        uint8_t *cq = malloc(M * H), *cs = malloc(M * H / 32);
        down(ch, dh2, 2 * M * H); down(cn, dn2, 2 * M * H); down(cq, dq2, M * H); down(cs, ds2, M * H / 32);
        if (memcmp(ch, gh, 2 * M * H) || memcmp(cn, gn, 2 * M * H) || memcmp(cq, gq, M * H) || memcmp(cs, gs, M * H / 32))
            FAIL("unfused chain (copy-only norm -> fp8_quant) differs from the fused launch");
        printf("unfused chain (copy-only norm -> fp8_quant): bit-identical to the fused launch\n");
        CHECK_HIP(hipFree(dh2)); CHECK_HIP(hipFree(dn2)); CHECK_HIP(hipFree(dq2)); CHECK_HIP(hipFree(ds2));
        free(ch); free(cn); free(cq); free(cs);

        CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dr)); CHECK_HIP(hipFree(dw)); CHECK_HIP(hipFree(dh));
        CHECK_HIP(hipFree(dq)); CHECK_HIP(hipFree(ds)); CHECK_HIP(hipFree(dn));
        free(x); free(r); free(w); free(gh); free(gn); free(oh); free(on); free(gq); free(gs); free(oq); free(os);
    }

    /* ---- SiLU-and-mul + 1x128, M = 20, I = 3072 (bit-identical to the oracle) */
    {
        const int64_t M = 20, I = 3072;
        uint16_t *gu = malloc(4 * M * I);
        for (int64_t i = 0; i < 2 * M * I; ++i) gu[i] = to_bf16((float)(3.0 * normal()));
        void *dg = dmalloc(4 * M * I), *dq = dmalloc(M * I), *ds = dmalloc(4 * M * (I / 128)), *da = dmalloc(2 * M * I);
        up(dg, gu, 4 * M * I);
        afq_act_desc d;
        memset(&d, 0, sizeof d);
        d.M = M; d.I = I; d.gate_up = dg; d.gate_up_row_stride = 2 * I; d.mode = AFQ_BLOCK128;
        d.quant_input = AFQ_QIN_DEFAULT;
        d.out.values = dq; d.out.scales = ds; d.out.normed = da;
        int stt = silu_mul_quant(&d, st);
        if (stt != AFQ_OK) FAIL("silu_mul_quant: %s", afq_status_string(stt));
        CHECK_HIP(hipStreamSynchronize(st));
        uint8_t *gq = malloc(M * I), *oq = malloc(M * I);
        float *gs = malloc(4 * M * (I / 128)), *os = malloc(4 * M * (I / 128));
        uint16_t *ga = malloc(2 * M * I), *oa = malloc(2 * M * I);
        down(gq, dq, M * I); down(gs, ds, 4 * M * (I / 128)); down(ga, da, 2 * M * I);
        orc_silu_quant_rows(M, I, gu, 2 * I, 1, 0, oq, os, oa, 0, M, work);
        compare16("silu 1x128 bf16 activation", ga, oa, M * I, 1);
        if (memcmp(gq, oq, M * I) != 0) FAIL("silu 1x128 codes not bit-identical");
        if (memcmp(gs, os, 4 * M * (I / 128)) != 0) FAIL("silu 1x128 scales not bit-identical");
        printf("silu 1x128 codes and scales: bit-identical (%lld elements)\n", (long long)(M * I));
        CHECK_HIP(hipFree(dg)); CHECK_HIP(hipFree(dq)); CHECK_HIP(hipFree(ds)); CHECK_HIP(hipFree(da));
        free(gu); free(gq); free(oq); free(gs); free(os); free(ga); free(oa);
    }

    /* ---- clamped SwiGLU (alpha 1.702, beta 1, limit 7) + MXFP8, M = 24, I = 768,
     *      gate_up ~ N(0, 8^2) */
    {
        const int64_t M = 24, I = 768;
        uint16_t *gu = malloc(4 * M * I);
        for (int64_t i = 0; i < 2 * M * I; ++i) gu[i] = to_bf16((float)(8.0 * normal()));
        void *dg = dmalloc(4 * M * I), *dq = dmalloc(M * I), *ds = dmalloc(M * (I / 32)), *da = dmalloc(2 * M * I);
        up(dg, gu, 4 * M * I);
        afq_swiglu_desc d;
        memset(&d, 0, sizeof d);
        d.act.M = M; d.act.I = I; d.act.gate_up = dg; d.act.gate_up_row_stride = 2 * I;
        d.act.mode = AFQ_MXFP8; d.act.quant_input = AFQ_QIN_DEFAULT;
        d.act.out.values = dq; d.act.out.scales = ds; d.act.out.normed = da;
        d.alpha = 1.702f; d.beta = 1.0f; d.limit = 7.0f;
        int stt = swiglu_oai_quant(&d, st);
        if (stt != AFQ_OK) FAIL("swiglu_oai_quant: %s", afq_status_string(stt));
        d.limit = 0.0f;
        if (swiglu_oai_quant(&d, st) != AFQ_ERR_ARG) FAIL("limit 0 not rejected");
        CHECK_HIP(hipStreamSynchronize(st));
        uint8_t *gq = malloc(M * I), *oq = malloc(M * I), *gs = malloc(M * (I / 32)), *os = malloc(M * (I / 32));
        uint16_t *ga = malloc(2 * M * I), *oa = malloc(2 * M * I);
        down(gq, dq, M * I); down(gs, ds, M * (I / 32)); down(ga, da, 2 * M * I);
        orc_swiglu_oai_quant_rows(M, I, gu, 2 * I, 0, 0, 1.702f, 1.0f, 7.0f, oq, os, oa, 0, M, work);
        compare16("swiglu MXFP8 bf16 activation", ga, oa, M * I, 0);
        compare_codes("swiglu MXFP8 codes", gq, oq, M * I);
        compare_bytes("swiglu E8M0 scales", gs, os, M * (I / 32), 1);
        CHECK_HIP(hipFree(dg)); CHECK_HIP(hipFree(dq)); CHECK_HIP(hipFree(ds)); CHECK_HIP(hipFree(da));
        free(gu); free(gq); free(oq); free(gs); free(os); free(ga); free(oa);
    }

    /* ---- standalone per-token quant of a strided fp32 [M, 2048] (bit-identical) */
    {
        const int64_t M = 50, n = 2048, stride = 2112;
        float *x = malloc(4 * M * stride);
        for (int64_t i = 0; i < M * stride; ++i) x[i] = (float)(normal() * exp2((double)(i / stride % 16) - 8));
        void *dx = dmalloc(4 * M * stride), *dq = dmalloc(M * n), *ds = dmalloc(4 * M);
        up(dx, x, 4 * M * stride);
        afq_quant_desc d;
        memset(&d, 0, sizeof d);
        d.M = M; d.cols = n; d.x = dx; d.x_row_stride = stride; d.dtype = AFQ_FP32; d.mode = AFQ_PER_TOKEN;
        d.out.values = dq; d.out.scales = ds;
        int stt = fp8_quant(&d, st);
        if (stt != AFQ_OK) FAIL("fp8_quant: %s", afq_status_string(stt));
        CHECK_HIP(hipStreamSynchronize(st));
        uint8_t *gq = malloc(M * n), *oq = malloc(M * n);
        float *gs = malloc(4 * M), *os = malloc(4 * M);
        down(gq, dq, M * n); down(gs, ds, 4 * M);
        orc_quant_rows(M, n, x, stride, 2, 2, oq, os, 0, M, work);
        if (memcmp(gq, oq, M * n) != 0 || memcmp(gs, os, 4 * M) != 0) FAIL("per-token quant not bit-identical");
        printf("per-token quant of strided fp32 rows: bit-identical (%lld elements)\n", (long long)(M * n));
        CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dq)); CHECK_HIP(hipFree(ds));
        free(x); free(gq); free(oq); free(gs); free(os);
    }

    CHECK_HIP(hipStreamDestroy(st));
    free(work);
    printf("c example ok\n");
    return 0;
}
