/* Runs the oracle's entry points on small inputs (every variant, ragged and minimal
 * shapes, a non-finite row, traces on and off) and on invalid arguments, under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "ok" and exits 0 when every
 * call returns its documented status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_any4_quantize_v(const void* w, int32_t dtype, int64_t n_rows, int64_t n_cols,
                           const float* act, int64_t row_offset, int32_t matrix_index,
                           int32_t group, int32_t n_clusters, int32_t iters, uint64_t seed,
                           int32_t variant, uint8_t* codes, uint16_t* lut, uint16_t* scale,
                           uint16_t* offset, double* objective, float* c_trace, double* j_trace,
                           int32_t* picks, float* c_final);
int oracle_act_absmean(const void* x, int32_t dtype, int64_t T, int64_t K, float* out);
int oracle_dequantize(const uint8_t* codes, const uint16_t* lut, const uint16_t* scale,
                      const uint16_t* offset, int64_t N, int64_t K, int32_t group, int32_t k,
                      float* out);
int oracle_lut_gemv(const uint8_t* codes, const uint16_t* lut, const uint16_t* scale,
                    const uint16_t* offset, int64_t N, int64_t K, int32_t group, int32_t k,
                    const void* x, int32_t dtype, int64_t M, float* y, double* s);
void oracle_fp16_rne_array(const float* in, uint16_t* out, int64_t n);
void oracle_bf16_rne_array(const float* in, uint16_t* out, int64_t n);
float oracle_fp16_to_f32(uint16_t h);

static int failures = 0;
#define EXPECT(expr, want)                                                        \
    do {                                                                          \
        int got_ = (expr);                                                        \
        if (got_ != (want)) {                                                     \
            fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #expr, got_, want); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static uint64_t lcg = 12345;
static float urand(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((lcg >> 40) & 0xFFFFFF) / 16777216.0f;
}

static int run(int64_t N, int64_t K, int32_t g, int32_t k, int32_t iters, int32_t variant, int nan_row,
               int trace) {
    float* w = malloc(sizeof(float) * N * K);
    float* act = malloc(sizeof(float) * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = (urand() - 0.5f) * 0.04f;
    for (int64_t j = 0; j < K; ++j) act[j] = 0.5f + urand();
    if (nan_row >= 0 && nan_row < N) w[nan_row * K] = NAN;
    uint8_t* codes = malloc(N * K / 2);
    uint16_t* lut = malloc(2 * N * k);
    uint16_t* sc = malloc(2 * N * (K / g));
    uint16_t* of = malloc(2 * N * (K / g));
    double* obj = malloc(8 * N);
    float* ct = trace ? malloc(sizeof(float) * N * (iters + 1) * k) : NULL;
    double* jt = trace ? malloc(8 * N * (iters + 1)) : NULL;
    int32_t* pk = malloc(4 * N * k);
    float* cf = malloc(4 * N * k);
    int st = oracle_any4_quantize_v(w, 0, N, K, act, 7, 1, g, k, iters, 99, variant, codes, lut, sc, of,
                                    obj, ct, jt, pk, cf);
    if (st == 0 || st == 5) {
        float* deq = malloc(sizeof(float) * N * K);
        EXPECT(oracle_dequantize(codes, lut, sc, of, N, K, g, k, deq), 0);
        float x[2 * 1024];
        for (int i = 0; i < 2 * K && i < 2 * 1024; ++i) x[i] = urand() - 0.5f;
        if (K <= 1024) {
            float y[2 * 64];
            double s[2 * 64];
            if (N <= 64) EXPECT(oracle_lut_gemv(codes, lut, sc, of, N, K, g, k, x, 0, 2, y, s), 0);
        }
        free(deq);
    }
    free(w); free(act); free(codes); free(lut); free(sc); free(of); free(obj);
    free(ct); free(jt); free(pk); free(cf);
    return st;
}

int main(void) {
    const int32_t variants[] = {0, 1, 2, 1 << 2, 2 << 2, 3 << 2, 1 << 4, (1 << 4) | (3 << 2) | 2,
                                1 << 8, (2 << 8) | (1 << 2)};
    for (unsigned v = 0; v < sizeof(variants) / sizeof(variants[0]); ++v) {
        EXPECT(run(5, 96, 32, 4, 5, variants[v], -1, 1), 0);
        EXPECT(run(3, 1000, 8, 16, 3, variants[v], -1, v & 1), 0);
        EXPECT(run(4, 2, 2, 2, 2, variants[v], -1, 1), 0);
        EXPECT(run(6, 512, 128, 16, 0, variants[v], 2, 1), 5);
    }
    EXPECT(run(2, 512, 128, 16, 3, 3, -1, 0), 1);        /* weighting 3 is not a variant */
    EXPECT(run(2, 512, 128, 16, 3, 1 << 5, -1, 0), 1);   /* unknown bit */
    EXPECT(run(2, 511, 1, 16, 3, 0, -1, 0), 1);          /* odd K */
    EXPECT(run(2, 512, 128, 3, 3, 0, -1, 0), 1);         /* 3 clusters */

    float x[3 * 40];
    uint16_t xb[3 * 40];
    float out[40];
    for (int i = 0; i < 120; ++i) x[i] = urand() * 4.0f - 2.0f;
    oracle_bf16_rne_array(x, xb, 120);
    EXPECT(oracle_act_absmean(x, 0, 3, 40, out), 0);
    EXPECT(oracle_act_absmean(xb, 1, 3, 40, out), 0);
    EXPECT(oracle_act_absmean(x, 0, 0, 40, out), 1);
    uint16_t h[120];
    oracle_fp16_rne_array(x, h, 120);
    for (int i = 0; i < 65536; i += 97) (void)oracle_fp16_to_f32((uint16_t)i);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
