/*
 * w4a4_oracle.c -- CPU ORACLE FOR THE W4A4 + INT8-OUTLIER LINEAR LAYER.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product package loads, links or
 * calls this file. Only the tests, the smoke check in __graft_entry__ and the
 * cpu_baseline leg of bench.py may use it. It shares no code, header, table or
 * constant with the HIP path.
 *
 * Plain, slow and written to be checked by eye against the pages:
 *   [QUIK]  "QUIK: Towards End-to-End 4-Bit Inference on Generative Large
 *           Language Models", abstract: most weights and activations go to
 *           4 bits, a few outlier weights/activations stay in higher precision.
 *   [ATOM]  "Atom: Low-bit Quantization for Efficient and Accurate LLM Serving"
 *           (research summary page), Summary paragraph 2 (8-bit outlier
 *           channels after reordering, fine-grained group quantization,
 *           activation scales computed per input), Key points item 5
 *           (symmetric quantization, no zero-point cross terms), Interesting
 *           ideas I1 (outlier channels moved to the end as one contiguous
 *           block) and I3 (outliers kept in INT8).
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *   R1 INT4 codes use qmax = 7, INT8 codes qmax = 127 (symmetric absmax); the
 *      clamp range is [-qmax-1, qmax] although -qmax-1 is never produced.
 *   R2 round to nearest, ties to even, applied to the fp32 quotient x / s.
 *   R3 x / s is one correctly rounded fp32 division (no reciprocal).
 *   R4 scales are fp32: s = fl32(absmax / qmax).
 *   R5 an all-zero block has s = 0 and all codes 0.
 *   R6 the reorder is stable: ascending non-outlier channels, then ascending
 *      outlier channels. Groups are cut after the reorder, inside the
 *      non-outlier segment only; the outlier tail is one block.
 *   R7 the tail has one scale per row (token for X, output channel for W).
 *   R8 dequantized output y* is evaluated in fp64 and rounded to fp16 by the
 *      caller (fp64 -> fp16 round to nearest even).
 *   N1-N3 (RMSNorm in front of the quantizer): at w4o_rms_rstd_rows.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * All floating point here is IEEE binary32 / binary64 on x86-64 SSE (no x87
 * excess precision), so every fp32 division is correctly rounded.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below use (reported by the benchmark). */
int w4o_max_threads(void) { return omp_get_max_threads(); }

/* Outlier permutation: perm = ascending(j not in O) ++ ascending(j in O).
 * [ATOM] Interesting ideas I1; reading R6.
 * Returns 0, or -1 if an index is out of [0, K) or repeated. */
int w4o_make_perm(int32_t K, const int32_t *outlier_idx, int32_t n_out,
                  int32_t *perm)
{
    if (K < 0 || n_out < 0 || n_out > K)
        return -1;
    unsigned char *is_out = (unsigned char *)calloc((size_t)K + 1, 1);
    if (!is_out)
        return -1;
    for (int32_t i = 0; i < n_out; ++i) {
        int32_t c = outlier_idx[i];
        if (c < 0 || c >= K || is_out[c]) {
            free(is_out);
            return -1;
        }
        is_out[c] = 1;
    }
    int32_t pos = 0;
    for (int32_t j = 0; j < K; ++j)
        if (!is_out[j])
            perm[pos++] = j;
    for (int32_t j = 0; j < K; ++j)
        if (is_out[j])
            perm[pos++] = j;
    free(is_out);
    return 0;
}

/* Symmetric round-to-nearest quantization of one block of len values.
 * [ATOM] Summary paragraph 2 (dynamic scale per input) and Key points item 5
 * (symmetric); readings R1-R5. */
void w4o_quantize_block(const float *v, int32_t len, int32_t qmax,
                        int8_t *q, float *scale)
{
    float a = 0.0f;
    for (int32_t j = 0; j < len; ++j) {
        float m = fabsf(v[j]);
        if (m > a)
            a = m;
    }
    float s = a / (float)qmax;
    *scale = s;
    for (int32_t j = 0; j < len; ++j) {
        if (s == 0.0f) {
            q[j] = 0;
            continue;
        }
        float r = rintf(v[j] / s);
        if (r > (float)qmax)
            r = (float)qmax;
        if (r < (float)(-qmax - 1))
            r = (float)(-qmax - 1);
        q[j] = (int8_t)r;
    }
}

/* RMSNorm factor of each row of a [rows, K] matrix of fp16 values (given
 * widened to fp32, row pitch ld floats), for the norm that precedes the
 * quantizer when the two are fused. [ATOM] Summary paragraph 2 (quantization
 * fused into the operators around the GEMM) and Interesting ideas I2; the
 * norm itself (mean square, eps, reciprocal square root) is the standard
 * RMSNorm of the Llama models the pages evaluate.
 * Readings (the pages give no arithmetic for the norm):
 *   N1 the sum of squares is exact: every x^2 * 2^48 is an integer below
 *      2^80 for fp16 x, so the sum of up to 2^15 of them is an integer below
 *      2^95, held in 128 bits;
 *   N2 rstd = fl32(1 / sqrt(fl64(fl64(S) / K) + eps)), each step one correctly
 *      rounded IEEE binary64 operation (S rounded to binary64 once);
 *   N3 a row whose mean square plus eps is zero (all zeros, eps = 0) has
 *      rstd = 0, so it normalizes to zeros.
 * Returns 0, or -1 for K <= 0 or K > 2^15 or eps negative or not finite. */
int w4o_rms_rstd_rows(const float *X, int64_t rows, int32_t K, int64_t ld, float eps,
                      float *rstd)
{
    if (K <= 0 || K > 32768 || !(eps >= 0.0f) || !isfinite(eps))
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        unsigned __int128 S = 0;
        for (int32_t j = 0; j < K; ++j) {
            double x = (double)X[r * ld + j];
            S += (unsigned __int128)(x * x * 0x1p48);
        }
        double d = (double)S * 0x1p-48;
        double v = d / (double)K + (double)eps;
        rstd[r] = v == 0.0 ? 0.0f : (float)(1.0 / sqrt(v));
    }
    return 0;
}

/* Number of INT4 scale groups per row: G = K_n / group, or 1 for one scale per
 * row, or 0 when every channel is an outlier. */
int32_t w4o_num_groups(int32_t K_n, int32_t group)
{
    if (K_n == 0)
        return 0;
    return group > 0 ? K_n / group : 1;
}

/* Reorder and quantize rows of a [rows, K] matrix (row pitch ld floats).
 * Outputs one code per byte (unpacked):
 *   q4 [rows, K_n] INT4 codes, s4 [rows, G] fp32 scales,
 *   q8 [rows, n_out] INT8 codes, s8 [rows] fp32 scales (0 when n_out == 0).
 * The same routine serves activations (rows = tokens) and weights
 * (rows = output channels): [QUIK] abstract keeps outliers of both.
 * Returns 0, or -1 when group does not divide K_n. */
int w4o_quantize_rows(const float *X, int64_t rows, int32_t K, int64_t ld,
                      const int32_t *perm, int32_t n_out, int32_t group,
                      int8_t *q4, float *s4, int8_t *q8, float *s8)
{
    int32_t K_n = K - n_out;
    if (n_out < 0 || K_n < 0 || group < 0 || (group > 0 && K_n % group != 0))
        return -1;
    int32_t G = w4o_num_groups(K_n, group);
    int32_t gl = group > 0 ? group : K_n;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float *xr = (float *)malloc(sizeof(float) * ((size_t)K + 1));
        for (int32_t j = 0; j < K; ++j)
            xr[j] = X[r * ld + perm[j]];
        for (int32_t t = 0; t < G; ++t)
            w4o_quantize_block(xr + (int64_t)t * gl, gl, 7,
                               q4 + r * K_n + (int64_t)t * gl, s4 + r * G + t);
        if (n_out > 0)
            w4o_quantize_block(xr + K_n, n_out, 127, q8 + r * n_out, s8 + r);
        else
            s8[r] = 0.0f;
        free(xr);
    }
    return 0;
}

/* Two's-complement nibble packing, two codes per byte, low nibble first:
 * byte(r, i) = (q[r, 2i] & 0xF) | (q[r, 2i+1] & 0xF) << 4, zero padding up to
 * pitch bytes. [QUIK] code samples name pack_to_i4 / two_compl (names only). */
void w4o_pack_nibbles(const int8_t *q, int64_t rows, int32_t K_n, int64_t pitch,
                      uint8_t *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        memset(out + r * pitch, 0, (size_t)pitch);
        for (int32_t j = 0; j < K_n; ++j) {
            uint8_t nib = (uint8_t)q[r * K_n + j] & 0x0F;
            out[r * pitch + j / 2] |= (uint8_t)(j % 2 == 0 ? nib : nib << 4);
        }
    }
}

/* The hybrid linear layer at selected output positions (m[p], n[p]).
 * For each pair p:
 *   acc4[p, t] = sum_{j in block t} qa4[m, j] * qw4[n, j]      (int64, exact)
 *   acc8[p]    = sum_{j < n_out}    qa8[m, j] * qw8[n, j]
 *   y[p] = sum_t sa4[m,t] sw4[n,t] acc4[p,t] + sa8[m] sw8[n] acc8[p]   (fp64)
 * [ATOM] Summary paragraph 2 (INT4 part plus 8-bit outlier part) and Key
 * points item 5 (symmetric scales factor out of the integer sums).
 * Scales are [rows, G] row-major. Returns 0, or -1 if an accumulator leaves
 * the int32 range. */
int w4o_linear_at(const int8_t *qa4, const float *sa4, const int8_t *qa8,
                  const float *sa8, const int8_t *qw4, const float *sw4,
                  const int8_t *qw8, const float *sw8, int32_t K_n,
                  int32_t n_out, int32_t group, const int32_t *m_idx,
                  const int32_t *n_idx, int64_t npairs, int32_t *acc4,
                  int32_t *acc8, double *y)
{
    int32_t G = w4o_num_groups(K_n, group);
    int32_t gl = group > 0 ? group : K_n;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t m = m_idx[p], n = n_idx[p];
        double yp = 0.0;
        for (int32_t t = 0; t < G; ++t) {
            int64_t s = 0;
            for (int32_t j = t * gl; j < (t + 1) * gl; ++j)
                s += (int64_t)qa4[m * K_n + j] * (int64_t)qw4[n * K_n + j];
            if (s > INT32_MAX || s < INT32_MIN)
                bad = 1;
            acc4[p * G + t] = (int32_t)s;
            yp += (double)sa4[m * G + t] * (double)sw4[n * G + t] * (double)s;
        }
        int64_t s8 = 0;
        for (int32_t j = 0; j < n_out; ++j)
            s8 += (int64_t)qa8[m * n_out + j] * (int64_t)qw8[n * n_out + j];
        if (s8 > INT32_MAX || s8 < INT32_MIN)
            bad = 1;
        acc8[p] = (int32_t)s8;
        yp += (double)sa8[m] * (double)sw8[n] * (double)s8;
        y[p] = yp;
    }
    return bad ? -1 : 0;
}

/* W4A8 layer (the QQQ abstract on the "smoothquant" tag page: 4-bit weights, 8-bit activations, per-channel
 * and per-group GEMMs) at selected output positions (m[p], n[p]):
 *   acc[p, t] = sum_{j in block t} qa8[m, j] * qw4[n, j]       (int64, exact)
 *   y[p] = sa8[m] * sum_t sw4[n, t] * acc[p, t]                 (fp64)
 * qa8 [M, K] INT8 codes with one scale per token (sa8 [M]); qw4 [N, K] INT4
 * codes with G = K / group scale groups per output channel (one when group
 * is 0). Returns 0, or -1 if an accumulator leaves the int32 range. */
int w4o_w4a8_linear_at(const int8_t *qa8, const float *sa8, const int8_t *qw4,
                       const float *sw4, int32_t K, int32_t group,
                       const int32_t *m_idx, const int32_t *n_idx, int64_t npairs,
                       int32_t *acc, double *y)
{
    int32_t G = w4o_num_groups(K, group);
    int32_t gl = group > 0 ? group : K;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t m = m_idx[p], n = n_idx[p];
        double yp = 0.0;
        for (int32_t t = 0; t < G; ++t) {
            int64_t s = 0;
            for (int32_t j = t * gl; j < (t + 1) * gl; ++j)
                s += (int64_t)qa8[m * K + j] * (int64_t)qw4[n * K + j];
            if (s > INT32_MAX || s < INT32_MIN)
                bad = 1;
            acc[p * G + t] = (int32_t)s;
            yp += (double)sw4[n * G + t] * (double)s;
        }
        y[p] = (double)sa8[m] * yp;
    }
    return bad ? -1 : 0;
}
