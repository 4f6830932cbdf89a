/* sanitize_check.c -- test infrastructure: runs every entry point of the CPU
 * oracle (fgfp8_oracle.c, included below) on ragged shapes with exactly sized
 * heap buffers, so that a build with -fsanitize=address,undefined reports any
 * out-of-bounds access, leak or undefined behaviour in the oracle itself.
 * Built and run by tests/test_oracle_sanitizers.py; not part of the product. */
#include "fgfp8_oracle.c"
#include <stdio.h>
#include <stdlib.h>

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng; }
static float frand(void) { return ((float)(next() >> 8) / 16777216.0f - 0.5f) * 4.0f; }
static uint16_t bf16(float f) { uint32_t b; memcpy(&b, &f, 4); return (uint16_t)(b >> 16); }

static void run_tok(int rows0, int cols0, int dtype, int gran, int fmt, int transpose) {
    int64_t n = (int64_t)rows0 * cols0, rows, cols, xs_row, xs_col, groups, units, g;
    void *x = malloc(n * (dtype ? 4 : 2));
    for (int64_t i = 0; i < n; ++i) {
        float v = frand();
        if (i % 977 == 0) v *= 1e4f;
        if (i < cols0) v = 0.0f;   /* an all-zero first row */
        if (dtype) ((float *)x)[i] = v; else ((uint16_t *)x)[i] = bf16(v);
    }
    if (transpose) { rows = cols0; cols = rows0; xs_row = 1; xs_col = cols0; }
    else { rows = rows0; cols = cols0; xs_row = cols0; xs_col = 1; }
    groups = (cols + gran - 1) / gran;
    units = fmt == ORC_SF_PACKED_UE8M0 ? (groups + 3) / 4 : groups;
    uint8_t *q = malloc(rows * cols);
    void *sf = malloc(rows * units * 4);
    /* row-major scales, then MN-major */
    if (orc_cast_per_token(x, dtype, rows, cols, xs_row, xs_col, gran, fmt, q, cols, sf, units, 1)) abort();
    if (orc_cast_per_token(x, dtype, rows, cols, xs_row, xs_col, gran, fmt, q, cols, sf, 1, rows)) abort();
    (void)g;
    free(x); free(q); free(sf);
}

static void run_blk(int rows, int cols, int dtype, int fmt) {
    int64_t n = (int64_t)rows * cols, br = (rows + 127) / 128, bc = (cols + 127) / 128;
    void *x = malloc(n * (dtype ? 4 : 2));
    for (int64_t i = 0; i < n; ++i) {
        float v = frand();
        if (dtype) ((float *)x)[i] = v; else ((uint16_t *)x)[i] = bf16(v);
    }
    uint8_t *q = malloc(n);
    float *sf = malloc(br * bc * 4);
    if (orc_cast_per_block(x, dtype, rows, cols, cols, fmt, q, cols, sf, bc)) abort();
    free(x); free(q); free(sf);
}

static void run_gemm(int m, int n, int k, int rows_per_scale, int sampled) {
    int kb = k / 128, nb = rows_per_scale == 128 ? (n + 127) / 128 : n;
    uint8_t *A = malloc((size_t)m * k), *B = malloc((size_t)n * k);
    float *sa = malloc((size_t)m * kb * 4), *sb = malloc((size_t)nb * kb * 4);
    for (int64_t i = 0; i < (int64_t)m * k; ++i) A[i] = (uint8_t)(next() >> 24) & 0xF7;
    for (int64_t i = 0; i < (int64_t)n * k; ++i) B[i] = (uint8_t)(next() >> 24) & 0xF7;
    for (int64_t i = 0; i < (int64_t)m * kb; ++i) sa[i] = 0.5f + (float)(next() % 100) / 100.0f;
    for (int64_t i = 0; i < (int64_t)nb * kb; ++i) sb[i] = 0.5f + (float)(next() % 100) / 100.0f;
    if (!sampled) {
        double *ref = malloc((size_t)m * n * 8), *abs_ = malloc((size_t)m * n * 8);
        if (orc_gemm_nt(A, k, sa, kb, 1, B, k, sb, kb, 1, rows_per_scale, m, n, k, NULL, NULL, 0, ref, abs_)) abort();
        free(ref); free(abs_);
    } else {
        int64_t cnt = 1000, *ii = malloc(cnt * 8), *jj = malloc(cnt * 8);
        double *ref = malloc(cnt * 8);
        for (int64_t o = 0; o < cnt; ++o) { ii[o] = next() % m; jj[o] = next() % n; }
        ii[0] = m - 1; jj[0] = n - 1;
        if (orc_gemm_nt(A, k, sa, kb, 1, B, k, sb, kb, 1, rows_per_scale, m, n, k, ii, jj, cnt, ref, NULL)) abort();
        free(ii); free(jj); free(ref);
    }
    free(A); free(B); free(sa); free(sb);
}

int main(void) {
    static const int shapes[][2] = {{1, 512}, {7, 4096}, {129, 7168}, {64, 1000}, {300, 257}, {5, 3}, {130, 33}};
    for (int s = 0; s < 7; ++s)
        for (int dt = 0; dt < 2; ++dt)
            for (int gi = 0; gi < 2; ++gi)
                for (int fmt = 0; fmt < 3; ++fmt)
                    for (int tr = 0; tr < 2; ++tr)
                        run_tok(shapes[s][0], shapes[s][1], dt, gi ? 128 : 32, fmt, tr);
    for (int s = 0; s < 7; ++s)
        for (int dt = 0; dt < 2; ++dt)
            for (int fmt = 0; fmt < 2; ++fmt) run_blk(shapes[s][0], shapes[s][1], dt, fmt);
    run_gemm(129, 200, 256, 128, 0);
    run_gemm(3, 300, 384, 1, 0);
    run_gemm(257, 130, 640, 128, 1);
    run_gemm(250, 38360, 384, 1, 1);
    {
        float v[4096]; uint8_t c[4096]; double d[4096]; uint16_t h[4096];
        for (int i = 0; i < 4096; ++i) { uint32_t b = next(); memcpy(&v[i], &b, 4); if (v[i] != v[i]) v[i] = 0; }
        orc_e4m3_round_array(v, 4096, c);
        orc_e4m3_value_array(c, 4096, d);
        orc_round_bf16_array(d, 4096, h);
    }
    orc_set_threads(2);
    printf("oracle under ASan/UBSan: all entry points ran clean (max threads %d)\n", orc_max_threads());
    return 0;
}
