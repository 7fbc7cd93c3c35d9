/* Drives every function of the C oracle on small inputs, edge cases included
 * (no outliers, every channel an outlier, all-zero blocks, group scales,
 * extreme values), for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer. Exit status 0 when every call returned what its
 * definition fixes; the sanitizers abort on the first memory or UB error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int w4o_max_threads(void);
int w4o_make_perm(int32_t K, const int32_t *outlier_idx, int32_t n_out, int32_t *perm);
void w4o_quantize_block(const float *v, int32_t len, int32_t qmax, int8_t *q, float *scale);
int w4o_rms_rstd_rows(const float *X, int64_t rows, int32_t K, int64_t ld, float eps, float *rstd);
int32_t w4o_num_groups(int32_t K_n, int32_t group);
int w4o_quantize_rows(const float *X, int64_t rows, int32_t K, int64_t ld, const int32_t *perm,
                      int32_t n_out, int32_t group, int8_t *q4, float *s4, int8_t *q8, float *s8);
void w4o_pack_nibbles(const int8_t *q, int64_t rows, int32_t K_n, int64_t pitch, uint8_t *out);
int w4o_linear_at(const int8_t *qa4, const float *sa4, const int8_t *qa8, const float *sa8,
                  const int8_t *qw4, const float *sw4, const int8_t *qw8, const float *sw8,
                  int32_t K_n, int32_t n_out, int32_t group, const int32_t *m_idx,
                  const int32_t *n_idx, int64_t npairs, int32_t *acc4, int32_t *acc8, double *y);
int w4o_w4a8_linear_at(const int8_t *qa8, const float *sa8, const int8_t *qw4, const float *sw4,
                       int32_t K, int32_t group, const int32_t *m_idx, const int32_t *n_idx,
                       int64_t npairs, int32_t *acc, double *y);

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

static uint32_t rng = 12345u;
static float uniform(void) { rng = rng * 1664525u + 1013904223u; return (float)(rng >> 8) / 16777216.0f * 2.0f - 1.0f; }

/* one layer case: rows x K activations and weights, n_out outliers, group */
static void layer_case(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group, float big) {
    const int32_t K_n = K - n_out;
    int32_t *outl = malloc(sizeof(int32_t) * (n_out > 0 ? n_out : 1));
    for (int32_t i = 0; i < n_out; ++i)
        outl[i] = (int32_t)((int64_t)i * K / (n_out > 0 ? n_out : 1));
    int32_t *perm = malloc(sizeof(int32_t) * K);
    CHECK(w4o_make_perm(K, outl, n_out, perm) == 0);
    float *X = malloc(sizeof(float) * M * K), *W = malloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < (int64_t)M * K; ++i) X[i] = uniform() * (i % 17 == 0 ? big : 1.0f);
    for (int64_t i = 0; i < (int64_t)N * K; ++i) W[i] = uniform() * 0.02f;
    for (int32_t j = 0; j < K; ++j) X[j] = 0.0f;                 /* an all-zero row */
    const int32_t G = w4o_num_groups(K_n, group);
    int8_t *qa4 = malloc(M * (K_n + 1)), *qw4 = malloc(N * (K_n + 1));
    int8_t *qa8 = malloc(M * (n_out + 1)), *qw8 = malloc(N * (n_out + 1));
    float *sa4 = malloc(sizeof(float) * M * (G + 1)), *sw4 = malloc(sizeof(float) * N * (G + 1));
    float *sa8 = malloc(sizeof(float) * M), *sw8 = malloc(sizeof(float) * N);
    CHECK(w4o_quantize_rows(X, M, K, K, perm, n_out, group, qa4, sa4, qa8, sa8) == 0);
    CHECK(w4o_quantize_rows(W, N, K, K, perm, n_out, group, qw4, sw4, qw8, sw8) == 0);
    for (int64_t i = 0; i < (int64_t)M * K_n; ++i) CHECK(qa4[i] >= -8 && qa4[i] <= 7);
    for (int32_t t = 0; t < G; ++t) CHECK(sa4[t] == 0.0f);      /* the zero row */
    const int64_t pitch = ((K_n + 127) / 128) * 64;
    uint8_t *packed = malloc(M * (pitch + 1));
    w4o_pack_nibbles(qa4, M, K_n, pitch, packed);
    int32_t m_idx[4] = {0, 1, M - 1, M / 2}, n_idx[4] = {0, N - 1, 1, N / 2};
    int32_t *acc4 = malloc(sizeof(int32_t) * 4 * (G + 1)), acc8[4];
    double y[4];
    CHECK(w4o_linear_at(qa4, sa4, qa8, sa8, qw4, sw4, qw8, sw8, K_n, n_out, group, m_idx, n_idx, 4,
                        acc4, acc8, y) == 0);
    CHECK(y[0] == 0.0);                                           /* row 0 is zero */
    float *rstd = malloc(sizeof(float) * M);
    CHECK(w4o_rms_rstd_rows(X, M, K, K, 1e-6f, rstd) == 0);
    CHECK(rstd[0] == (float)(1.0 / sqrt(1e-6f)));
    free(outl); free(perm); free(X); free(W); free(qa4); free(qw4); free(qa8); free(qw8);
    free(sa4); free(sw4); free(sa8); free(sw8); free(packed); free(acc4); free(rstd);
}

int main(void) {
    CHECK(w4o_max_threads() >= 1);
    int32_t perm[16], bad[2] = {3, 3}, out_of_range[1] = {16};
    CHECK(w4o_make_perm(16, bad, 2, perm) == -1);
    CHECK(w4o_make_perm(16, out_of_range, 1, perm) == -1);
    CHECK(w4o_make_perm(16, NULL, 0, perm) == 0 && perm[15] == 15);
    CHECK(w4o_make_perm(0, NULL, 0, perm) == 0);
    CHECK(w4o_num_groups(0, 0) == 0 && w4o_num_groups(256, 128) == 2 && w4o_num_groups(240, 0) == 1);

    float zeros[8] = {0}, s = -1.0f;
    int8_t q[8];
    w4o_quantize_block(zeros, 8, 7, q, &s);
    CHECK(s == 0.0f && q[0] == 0 && q[7] == 0);
    float ext[4] = {65504.0f, -65504.0f, 1e-7f, -0.0f};
    w4o_quantize_block(ext, 4, 127, q, &s);
    CHECK(q[0] == 127 && q[1] == -127 && q[2] == 0);
    CHECK(w4o_quantize_rows(zeros, 1, 8, 8, perm, 0, 3, q, &s, q, &s) == -1);   /* group does not divide */

    layer_case(9, 7, 300, 44, 128, 40.0f);     /* group scales, ragged rows */
    layer_case(5, 3, 257, 1, 0, 100.0f);       /* one scale per row, odd K */
    layer_case(4, 4, 64, 0, 0, 1.0f);          /* no outliers */
    layer_case(3, 2, 32, 32, 0, 50.0f);        /* every channel an outlier (K_n = 0) */

    int8_t qa8[2 * 256], qw4[3 * 256];
    float sa8[2] = {0.5f, 0.25f}, sw4[3 * 2] = {1, 2, 3, 4, 5, 6};
    for (int i = 0; i < 2 * 256; ++i) qa8[i] = (int8_t)((i * 37) % 255 - 127);
    for (int i = 0; i < 3 * 256; ++i) qw4[i] = (int8_t)((i * 11) % 16 - 8);
    int32_t mi[2] = {0, 1}, ni[2] = {2, 0}, acc[4];
    double yy[2];
    CHECK(w4o_w4a8_linear_at(qa8, sa8, qw4, sw4, 256, 128, mi, ni, 2, acc, yy) == 0);
    CHECK(w4o_w4a8_linear_at(qa8, sa8, qw4, sw4, 256, 0, mi, ni, 2, acc, yy) == 0);

    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle sanitizer run: all checks passed\n");
    return failures ? 1 : 0;
}
