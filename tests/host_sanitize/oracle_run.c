/*
 * oracle_run.c -- runs every path of the CPU oracle (oracle/afq_oracle.c)
 * on random and edge-case rows, built with gcc -fsanitize=address,undefined,
 * so that an out-of-bounds access, a use of uninitialised table state or an
 * undefined operation anywhere in the oracle aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (C linkage, no header) */
int orc_quant_rows(int64_t M, int64_t n, const void *x, int64_t x_stride, int in_dtype,
                   int mode, uint8_t *values, void *scales, int64_t r0, int64_t r1, double *work);
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
uint16_t orc_round_bf16(double v);
uint16_t orc_round_fp16(double v);
uint8_t orc_round_e4m3(double v);
uint8_t orc_e8m0_byte(float amax);

static uint64_t st = 88172645463325252ull;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

/* a finite bf16 / fp16 bit pattern: mostly moderate values, sometimes any
 * finite pattern (tiny, huge, subnormal, zero of either sign) */
static uint16_t pat16(int fp16)
{
    for (;;) {
        uint16_t b = (uint16_t)next();
        uint16_t e = fp16 ? (b >> 10) & 0x1F : (b >> 7) & 0xFF;
        if (e == (fp16 ? 0x1F : 0xFF)) continue;
        if (next() % 4) {           /* moderate: exponent near the bias */
            if (fp16) b = (uint16_t)((b & 0x83FF) | ((uint16_t)(12 + next() % 6) << 10));
            else b = (uint16_t)((b & 0x807F) | ((uint16_t)(120 + next() % 12) << 7));
        }
        return b;
    }
}

static void fill(uint16_t *p, int64_t n, int fp16, int kind)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (kind) {
        case 0: p[i] = pat16(fp16); break;
        case 1: p[i] = 0; break;                                   /* all-zero row */
        case 2: p[i] = (uint16_t)(next() % 2 ? 0x8000 : 0); break; /* signed zeros */
        default: p[i] = (uint16_t)(next() % 0x80);                 /* subnormals */
        }
    }
}

int main(void)
{
    const int64_t widths[] = {32, 128, 256, 384, 2048};
    double *work = malloc(sizeof(double) * 2 * 32768);
    long rows_done = 0;
    for (int w = 0; w < 5; ++w) {
        const int64_t H = widths[w], M = 6;
        uint16_t *x = malloc(2 * M * H), *r = malloc(2 * M * H), *wt = malloc(2 * H);
        uint16_t *h = malloc(2 * M * H), *nrm = malloc(2 * M * H), *gu = malloc(4 * M * H);
        uint8_t *q = malloc(M * H);
        float *sc = malloc(4 * M * H); /* large enough for every mode */
        float *xf = malloc(4 * M * H);
        for (int dt = 0; dt < 2; ++dt) {
            for (int64_t i = 0; i < M; ++i) fill(x + i * H, H, dt, (int)(i % 4));
            fill(r, M * H, dt, 0);
            fill(wt, H, dt, 0);
            for (int mode = 0; mode < 3; ++mode) {
                if (mode == 0 && H % 32) continue;
                if (mode == 1 && H % 128) continue;
                for (int kind = 0; kind < 2; ++kind)
                    for (int qin = 0; qin < 2; ++qin)
                        for (int res = 0; res < 2; ++res) {
                            if (qin == 1 && mode == 0) continue;
                            int rc = orc_norm_quant_rows(M, H, x, H, res ? r : NULL, res ? h : NULL, wt, kind, dt,
                                                         mode, qin, 1e-6f, q, sc, nrm, 0, M, work);
                            if (rc != 0) { fprintf(stderr, "norm rc %d\n", rc); return 1; }
                            rows_done += M;
                        }
                int rc = orc_quant_rows(M, H, x, H, dt, mode, q, sc, 0, M, work);
                if (rc != 0) return 1;
            }
        }
        for (int64_t i = 0; i < M * H; ++i) xf[i] = (float)((int64_t)(next() % 2001) - 1000) * 0x1p-7f;
        xf[0] = 0.0f;
        xf[1] = -0.0f;
        xf[2] = 1e-40f;
        for (int mode = 0; mode < 3; ++mode) {
            if ((mode == 0 && H % 32) || (mode == 1 && H % 128)) continue;
            if (orc_quant_rows(M, H, xf, H, 2, mode, q, sc, 0, M, work) != 0) return 1;
        }
        for (int64_t i = 0; i < M; ++i) fill(gu + i * 2 * H, 2 * H, 0, (int)(i % 4));
        gu[0] = 0xC2C8; /* gate -100 */
        gu[1] = 0x42C8; /* gate +100 */
        for (int mode = 0; mode < 2; ++mode)
            for (int qin = 0; qin < 3; qin += 2) {
                if ((mode == 0 && H % 32) || (mode == 1 && H % 128)) continue;
                if (orc_silu_quant_rows(M, H, gu, 2 * H, mode, qin, q, sc, nrm, 0, M, work) != 0) return 1;
                rows_done += M;
            }
        if (orc_silu_quant_rows(M, H, gu, 2 * H, 2, 0, q, sc, nrm, 0, M, work) != -1) return 1; /* per-token */
        if (H % 32 == 0) {
            const float par[3][3] = {{1.702f, 1.0f, 7.0f}, {1.0f, 0.0f, INFINITY}, {-0.5f, -3.0f, 1e-3f}};
            for (int k = 0; k < 3; ++k)
                for (int qin = 0; qin < 3; qin += 2) {
                    if (orc_swiglu_oai_quant_rows(M, H, gu, 2 * H, 0, qin, par[k][0], par[k][1], par[k][2],
                                                  q, sc, nrm, 0, M, work) != 0) return 1;
                    rows_done += M;
                }
        }
        if (orc_swiglu_oai_quant_rows(M, H, gu, 2 * H, 1, 0, 1.702f, 1.0f, 7.0f, q, sc, nrm, 0, M, work) != -1)
            return 1; /* MXFP8 only */
        free(x); free(r); free(wt); free(h); free(nrm); free(gu); free(q); free(sc); free(xf);
    }
    /* the scalar format helpers at their boundaries */
    const double v[] = {0.0, -0.0, 448.0, 464.0, -464.0, 0x1p-10, 0x1p-9, 1e300, -1e300, 0x1p-1074};
    for (int i = 0; i < 10; ++i) {
        (void)orc_round_bf16(v[i]);
        (void)orc_round_fp16(v[i]);
        if (fabs(v[i]) <= 448.0) (void)orc_round_e4m3(v[i]);
    }
    const float a[] = {0.0f, 0x1p-149f, 0x1p-126f, 1.0f, 448.0f, 0x1.fffffep127f};
    for (int i = 0; i < 6; ++i) (void)orc_e8m0_byte(a[i]);
    free(work);
    printf("oracle paths ok (%ld rows)\n", rows_done);
    return 0;
}
