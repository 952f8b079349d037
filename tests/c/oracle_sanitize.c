/* Drives every entry point of the CPU oracle (oracle/qmm_oracle.c) on small seeded inputs, with
 * every buffer allocated at exactly the size the call needs, so that a build with
 * -fsanitize=address,undefined reports any read or write past a buffer, any signed overflow or
 * any other undefined behaviour in the oracle's host code.  Exit status 0 and a final "ok" line:
 * no finding (the sanitizers abort on the first one).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_half_to_double(uint16_t h);
uint16_t oracle_float_to_half(float x);
void oracle_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, uint8_t *y);
int64_t oracle_row_bytes(int type, int64_t k);
int64_t oracle_subdots_per_row(int type, int64_t k);
int oracle_dequantize(int type, const uint8_t *w, int64_t rows, int64_t k, double *out);
void oracle_dequantize_q8_1(const uint8_t *xq, int64_t n_rows, int64_t k, double *out, double *d_out, double *s_out);
int oracle_matmul_q8_1(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y);
int oracle_matmul_q8_1_at(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                          const int64_t *cols, const int64_t *rws, int64_t count, float *out);
int oracle_subdots(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, int32_t *D);
int oracle_subdots_q6_K_folded(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, int32_t *F);
int oracle_subdots_q3_K_folded(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, int32_t *F);
int oracle_matmul(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y);
int oracle_matmul_id(int type, const uint8_t *w, int64_t n_exp, int64_t rows, int64_t k, const float *x,
                     int64_t x_per_tok, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y,
                     int64_t *n_invalid);
int oracle_matmul_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const float *x,
                      int64_t n, float *y);
int oracle_matmul_id_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t n_exp, int64_t rows, int64_t k,
                         const float *x, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y,
                         int64_t *n_invalid);
int oracle_f16act_encode(const float *x, int64_t n, int64_t k, uint16_t *y, int32_t *e, double *bsum);
int oracle_matmul_f16act(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {   /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float rnd_normalish(void) { return ((float)(rnd() % 20001) - 10000.0f) / 3000.0f; }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static const int kTypes[] = {2, 8, 11, 12, 13, 14, 23};   /* Q4_0, Q8_0, Q3_K, Q4_K, Q5_K, Q6_K, IQ4_XS */

/* random block bytes with every fp16 field a finite value in [0.001, 0.02] */
static void fill_weights(int type, uint8_t *w, int64_t rows, int64_t k) {
    const int64_t rb = oracle_row_bytes(type, k);
    for (int64_t i = 0; i < rows * rb; ++i) w[i] = (uint8_t)rnd();
    const int qk = (type == 2 || type == 8) ? 32 : 256;
    const int bb = (int)(rb / (k / qk));
    for (int64_t b = 0; b < rows * (k / qk); ++b) {
        uint8_t *p = w + b * bb;
        uint16_t d = oracle_float_to_half(0.001f + 0.019f * (float)(rnd() % 1000) / 1000.0f);
        uint16_t m = oracle_float_to_half(0.001f + 0.019f * (float)(rnd() % 1000) / 1000.0f);
        if (type == 14) { memcpy(p + 208, &d, 2); }
        else if (type == 11) { memcpy(p + 108, &d, 2); }
        else { memcpy(p, &d, 2); if (type == 12 || type == 13) memcpy(p + 2, &m, 2); }
    }
}

static int run_type(int type, int64_t rows, int64_t k, int64_t n) {
    const int64_t rb = oracle_row_bytes(type, k), nb = k / 32;
    uint8_t *w = xmalloc((size_t)(rows * rb)), *w2 = xmalloc((size_t)(rows * rb));
    fill_weights(type, w, rows, k);
    fill_weights(type, w2, rows, k);
    float *x = xmalloc(sizeof(float) * (size_t)(n * k));
    for (int64_t i = 0; i < n * k; ++i) x[i] = rnd_normalish();
    if (n * k >= 64) { memset(x, 0, sizeof(float) * 32); x[40] = 1e30f; x[41] = -1e-40f; }   /* zero, huge, subnormal */
    uint8_t *xq = xmalloc((size_t)(n * nb * 36));
    oracle_quantize_q8_1(x, n, k, xq);
    double *deq = xmalloc(sizeof(double) * (size_t)(rows * k));
    if (oracle_dequantize(type, w, rows, k, deq)) return 1;
    double *xd = xmalloc(sizeof(double) * (size_t)(n * k)), *dd = xmalloc(sizeof(double) * (size_t)(n * nb)),
           *sd = xmalloc(sizeof(double) * (size_t)(n * nb));
    oracle_dequantize_q8_1(xq, n, k, xd, dd, sd);
    float *y = xmalloc(sizeof(float) * (size_t)(n * rows));
    if (oracle_matmul_q8_1(type, w, rows, k, xq, n, y)) return 1;
    if (oracle_matmul(type, w, rows, k, x, n, y)) return 1;
    if (oracle_matmul_glu(type, w, w2, rows, k, x, n, y)) return 1;
    const int64_t cnt = 17;
    int64_t cols[17], rws[17];
    for (int i = 0; i < cnt; ++i) { cols[i] = n ? (int64_t)(rnd() % (uint32_t)n) : 0; rws[i] = (int64_t)(rnd() % (uint32_t)rows); }
    float *at = xmalloc(sizeof(float) * (size_t)cnt);
    if (n && oracle_matmul_q8_1_at(type, w, rows, k, xq, n, cols, rws, cnt, at)) return 1;
    int32_t *D = xmalloc(sizeof(int32_t) * (size_t)(n * rows * oracle_subdots_per_row(type, k)));
    if (oracle_subdots(type, w, rows, k, xq, n, D)) return 1;
    if (type == 14 || type == 11) {
        int32_t *F = xmalloc(sizeof(int32_t) * (size_t)(n * rows * nb));
        if ((type == 14 ? oracle_subdots_q6_K_folded : oracle_subdots_q3_K_folded)(w, rows, k, xq, n, F)) return 1;
        free(F);
    }
    uint16_t *y16 = xmalloc(sizeof(uint16_t) * (size_t)(n * k));
    int32_t *e = xmalloc(sizeof(int32_t) * (size_t)(n * nb));
    double *bs = xmalloc(sizeof(double) * (size_t)(n * nb));
    if (oracle_f16act_encode(x, n, k, y16, e, bs)) return 1;
    if (n <= 8 && oracle_matmul_f16act(type, w, rows, k, x, n, y)) return 1;
    /* expert products: 3 experts, ids with invalid entries, per-slot and shared activations */
    const int64_t n_exp = 3, top_k = 2, n_tok = n;
    uint8_t *we = xmalloc((size_t)(n_exp * rows * rb)), *we2 = xmalloc((size_t)(n_exp * rows * rb));
    fill_weights(type, we, n_exp * rows, k);
    fill_weights(type, we2, n_exp * rows, k);
    int32_t *ids = xmalloc(sizeof(int32_t) * (size_t)(n_tok * top_k));
    for (int64_t i = 0; i < n_tok * top_k; ++i) ids[i] = (int32_t)(rnd() % 4) - (i % 7 == 3 ? 5 : 0);
    float *xe = xmalloc(sizeof(float) * (size_t)(n_tok * top_k * k));
    for (int64_t i = 0; i < n_tok * top_k * k; ++i) xe[i] = rnd_normalish();
    float *ye = xmalloc(sizeof(float) * (size_t)(n_tok * top_k * rows));
    int64_t bad = -1;
    if (oracle_matmul_id(type, we, n_exp, rows, k, xe, top_k, ids, n_tok, top_k, ye, &bad)) return 1;
    if (oracle_matmul_id(type, we, n_exp, rows, k, xe, 1, ids, n_tok, top_k, ye, &bad)) return 1;
    if (oracle_matmul_id_glu(type, we, we2, n_exp, rows, k, xe, ids, n_tok, top_k, ye, &bad)) return 1;
    free(w); free(w2); free(x); free(xq); free(deq); free(xd); free(dd); free(sd); free(y); free(at); free(D);
    free(y16); free(e); free(bs); free(we); free(we2); free(ids); free(xe); free(ye);
    return 0;
}

int main(void) {
    /* fp16 conversion over every pattern and a sweep of floats */
    for (uint32_t h = 0; h < 65536; ++h) (void)oracle_half_to_double((uint16_t)h);
    for (int i = 0; i < 100000; ++i) { uint32_t b = rnd(); float f; memcpy(&f, &b, 4); (void)oracle_float_to_half(f); }
    for (size_t t = 0; t < sizeof kTypes / sizeof kTypes[0]; ++t) {
        const int type = kTypes[t];
        const int64_t qk = (type == 2 || type == 8) ? 32 : 256;
        const int64_t shapes[][3] = {{1, qk, 1}, {7, 3 * qk, 5}, {33, 4 * qk, 9}, {5, qk, 0}};
        for (size_t s = 0; s < 4; ++s)
            if (run_type(type, shapes[s][0], shapes[s][1], shapes[s][2])) {
                fprintf(stderr, "oracle call failed: type %d shape %zu\n", type, s);
                return 1;
            }
    }
    /* argument errors are reported, not acted on */
    float yv[4];
    if (oracle_matmul_q8_1(12, NULL, 1, 100, NULL, 1, yv) == 0) return 1;
    if (oracle_matmul_q8_1(3, NULL, 1, 256, NULL, 1, yv) == 0) return 1;   /* unsupported type */
    printf("ok\n");
    return 0;
}
