/*
 * Sanitizer driver of the CPU oracle (test infrastructure): compiles
 * oracle/nvfp4_oracle.c into this translation unit with AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_oracle_sanitize.py)
 * and calls every exported function on small, ragged inputs: every block
 * kind and rule, a handed-in amax, a zero tensor, subnormal and saturating
 * values, the GEMM on 1D, 2D and COL16 operands, the sampled GEMM, the
 * random Hadamard transform, key smoothing and the exact-reading diagnostic.
 * Exit status 0 and no sanitizer report means every access stayed in bounds.
 */
#include "nvfp4_oracle.c"

#include <stdio.h>

static uint32_t lcg_state = 12345u;
static float next_uniform(void)   /* [-1, 1) */
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (float)((int32_t)(lcg_state >> 8) - (1 << 23)) / (float)(1 << 23);
}

static float *random_tensor(int64_t rows, int64_t cols, float scale)
{
    float *x = (float *)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(float));
    for (int64_t i = 0; i < rows * cols; i++)
        x[i] = next_uniform() * scale;
    return x;
}

static int quantize_all(const float *x, int64_t rows, int64_t cols, int block)
{
    int64_t nb;
    if (block == NVO_ROW16) nb = rows * (cols / 16);
    else if (block == NVO_TILE16) nb = (rows / 16) * (cols / 16);
    else nb = cols * (rows / 16);
    for (int rule = 0; rule < 2; rule++)
        for (int with_amax = 0; with_amax < 2; with_amax++) {
            uint8_t *codes = (uint8_t *)malloc((size_t)(rows * cols / 2 > 0 ? rows * cols / 2 : 1));
            uint8_t *scales = (uint8_t *)malloc((size_t)(nb > 0 ? nb : 1));
            float *y = (float *)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(float));
            float alpha;
            int64_t stats[2];
            float amax = 3.5f;
            nvo_quantize(x, rows, cols, cols, block, rule, with_amax ? &amax : NULL, codes, scales, &alpha,
                         stats);
            nvo_dequantize(codes, scales, alpha, rows, cols, block, y, cols);
            nvo_quantize_exact_reading(x, rows, cols, cols, block, rule, codes, scales, &alpha);
            free(codes);
            free(scales);
            free(y);
        }
    return 0;
}

int main(void)
{
    /* formats: every code and byte, values around every boundary */
    for (int c = 0; c < 16; c++)
        (void)nvo_e2m1_value(c);
    for (int b = 0; b < 127; b++)
        (void)nvo_e4m3_value(b);
    const float specials[] = {0.0f, -0.0f, 1e-45f, 1e-38f, 0.25f, 0.75f, 5.0f, 6.0f, 7.0f, 1e30f,
                              0x1p-10f, 0x1p-9f, 448.0f, 464.0f, 500.0f, 3e38f};
    for (unsigned i = 0; i < sizeof(specials) / sizeof(specials[0]); i++) {
        (void)nvo_e2m1_encode(specials[i]);
        (void)nvo_e2m1_encode(-specials[i]);
        (void)nvo_e4m3_encode(specials[i]);
        (void)nvo_global_scale(specials[i]);
    }

    /* quantize / dequantize / exact reading, every block kind, ragged sizes */
    float *a = random_tensor(5, 48, 3.0f);
    a[7] = 1e-40f;                            /* a subnormal element */
    quantize_all(a, 5, 48, NVO_ROW16);
    float *w = random_tensor(32, 48, 0.02f);
    quantize_all(w, 32, 48, NVO_TILE16);
    float *g = random_tensor(48, 7, 1e-3f);
    quantize_all(g, 48, 7, NVO_COL16);
    float *z = (float *)calloc(16 * 32, sizeof(float));
    quantize_all(z, 16, 32, NVO_ROW16);
    quantize_all(z, 16, 32, NVO_TILE16);
    quantize_all(z, 16, 32, NVO_COL16);
    quantize_all(a, 0, 48, NVO_ROW16);        /* empty */

    /* GEMM: A ROW16 [5][48] x B TILE16 [32][48]^T, and two COL16 operands */
    uint8_t ca[5 * 24], sa[5 * 3], cb[32 * 24], sb[2 * 3];
    float aa, ab;
    nvo_quantize(a, 5, 48, 48, NVO_ROW16, NVO_4OVER6, NULL, ca, sa, &aa, NULL);
    nvo_quantize(w, 32, 48, 48, NVO_TILE16, NVO_4OVER6, NULL, cb, sb, &ab, NULL);
    double c[5 * 32];
    if (nvo_gemm_f64(ca, sa, aa, 0, cb, sb, ab, 1, 5, 32, 48, c) != 0)
        return 2;
    int64_t ms[3] = {0, 4, 2}, ns[3] = {31, 0, 17};
    double cs[3];
    nvo_gemm_f64_sampled(ca, sa, aa, 0, cb, sb, ab, 1, 48, ms, ns, 3, cs);
    for (int i = 0; i < 3; i++)
        if (cs[i] != c[ms[i] * 32 + ns[i]])
            return 3;
    float *h = random_tensor(48, 9, 1.0f);
    uint8_t cg[7 * 24], sg[7 * 3], ch[9 * 24], sh[9 * 3];
    float ag, ah;
    nvo_quantize(g, 48, 7, 7, NVO_COL16, NVO_4OVER6, NULL, cg, sg, &ag, NULL);
    nvo_quantize_col16_rht(h, 48, 9, 9, NVO_4OVER6, 0x6D2Bu, NULL, ch, sh, &ah, NULL);
    double cw[7 * 9];
    if (nvo_gemm_f64(cg, sg, ag, 0, ch, sh, ah, 0, 7, 9, 48, cw) != 0)
        return 4;

    /* RHT and key smoothing */
    float v[16];
    for (int i = 0; i < 16; i++)
        v[i] = next_uniform();
    nvo_rht16(v, 0xFFFFu);
    float *k = random_tensor(9, 64, 2.0f);
    float *ks = (float *)malloc(9 * 64 * sizeof(float));
    float means[9];
    nvo_kv_smooth(k, 9, 64, ks, means);
    (void)nvo_amax(k, 9, 64, 64);
    (void)nvo_num_threads();

    free(a); free(w); free(g); free(z); free(h); free(k); free(ks);
    printf("oracle sanitizer driver ok\n");
    return 0;
}
