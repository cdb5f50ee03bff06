/*
 * Sanitizer driver for the CPU oracle (built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py, single-threaded).
 * Every buffer is allocated at exactly the size the oracle's layout needs,
 * so a read or write one element past any of them is reported.  Shapes:
 * ragged K (not a multiple of the scale group), ragged N, row subsets, the
 * empty and degenerate cases and the argument errors.  Each result is also
 * compared with a direct per-element evaluation of the definition here.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double a8w8_oracle_e4m3fn_value(uint8_t code);
double a8w8_oracle_e8m0_value(uint8_t code);
int a8w8_oracle_gemm(const uint8_t *A, const float *a_scale, const uint8_t *W, const float *w_scale, int64_t M,
                     int64_t N, int64_t K, const int64_t *rows, int64_t n_rows, double *Y);
int a8w8_oracle_gemm_mx(const uint8_t *A, const uint8_t *a_scale, const uint8_t *W, const uint8_t *w_scale, int64_t M,
                        int64_t N, int64_t K, const int64_t *rows, int64_t n_rows, double *Y);
int a8w8_oracle_gemm_rowwise(const uint8_t *A, const float *a_scale, const uint8_t *W, const float *w_scale,
                             int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t n_rows, double *Y);

static uint32_t rng = 12345u;
static uint32_t next(void)
{
    rng = rng * 1664525u + 1013904223u;
    return rng >> 8;
}
static uint8_t finite_code(void)
{
    uint8_t c = (uint8_t)next();
    return (c & 0x7F) == 0x7F ? 0x38 : c;   /* avoid NaN codes */
}

static int fails = 0;
#define CHECK(c, ...)                      \
    do {                                   \
        if (!(c)) {                        \
            fprintf(stderr, __VA_ARGS__);  \
            fprintf(stderr, "\n");         \
            ++fails;                       \
        }                                  \
    } while (0)

static void one(int kind, int64_t M, int64_t N, int64_t K, int subset)
{
    const int64_t G = kind == 1 ? 32 : 128;
    const int64_t KG = (K + G - 1) / G, NG = (N + G - 1) / G;
    uint8_t *A = malloc((size_t)(M * K) + 1), *W = malloc((size_t)(N * K) + 1);
    float *as = NULL, *ws = NULL;
    uint8_t *asb = NULL, *wsb = NULL;
    for (int64_t i = 0; i < M * K; ++i) A[i] = finite_code();
    for (int64_t i = 0; i < N * K; ++i) W[i] = finite_code();
    if (kind == 0) {
        as = malloc(sizeof(float) * (size_t)(M * KG) + 1);
        ws = malloc(sizeof(float) * (size_t)(NG * KG) + 1);
        for (int64_t i = 0; i < M * KG; ++i) as[i] = 0.5f + (float)(next() % 1000) / 1000.0f;
        for (int64_t i = 0; i < NG * KG; ++i) ws[i] = 0.001f * (1.0f + (float)(next() % 1000) / 1000.0f);
    } else if (kind == 1) {
        asb = malloc((size_t)(M * KG) + 1);
        wsb = malloc((size_t)(NG * KG) + 1);
        for (int64_t i = 0; i < M * KG; ++i) asb[i] = (uint8_t)(120 + next() % 10);
        for (int64_t i = 0; i < NG * KG; ++i) wsb[i] = (uint8_t)(120 + next() % 10);
    } else {
        as = malloc(sizeof(float) * (size_t)M + 1);
        ws = malloc(sizeof(float) * (size_t)N + 1);
        for (int64_t i = 0; i < M; ++i) as[i] = 0.5f + (float)(next() % 1000) / 1000.0f;
        for (int64_t i = 0; i < N; ++i) ws[i] = 0.01f;
    }
    int64_t n_rows = subset ? (M + 1) / 2 : M;
    int64_t *rows = NULL;
    if (subset) {
        rows = malloc(sizeof(int64_t) * (size_t)n_rows + 1);
        for (int64_t r = 0; r < n_rows; ++r) rows[r] = (r * 7 + 3) % M;
    }
    double *Y = malloc(sizeof(double) * (size_t)(n_rows * N) + 1);
    int rc = kind == 0 ? a8w8_oracle_gemm(A, as, W, ws, M, N, K, rows, n_rows, Y)
           : kind == 1 ? a8w8_oracle_gemm_mx(A, asb, W, wsb, M, N, K, rows, n_rows, Y)
                       : a8w8_oracle_gemm_rowwise(A, as, W, ws, M, N, K, rows, n_rows, Y);
    CHECK(rc == 0, "kind %d M=%lld N=%lld K=%lld: rc %d", kind, (long long)M, (long long)N, (long long)K, rc);
    for (int64_t r = 0; r < n_rows && rc == 0; ++r) {
        const int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            double want = 0.0, rw = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = a8w8_oracle_e4m3fn_value(A[m * K + k]) * a8w8_oracle_e4m3fn_value(W[n * K + k]);
                if (kind == 0)
                    want += p * (double)as[m * KG + k / G] * (double)ws[(n / G) * KG + k / G];
                else if (kind == 1)
                    want += p * a8w8_oracle_e8m0_value(asb[m * KG + k / G]) *
                            a8w8_oracle_e8m0_value(wsb[(n / G) * KG + k / G]);
                else
                    rw += p;
            }
            if (kind == 2)
                want = rw * (double)as[m] * (double)ws[n];
            const double got = Y[r * N + n];
            CHECK(fabs(got - want) <= 1e-9 * (1.0 + fabs(want)), "kind %d m=%lld n=%lld: %g vs %g", kind,
                  (long long)m, (long long)n, got, want);
        }
    }
    free(A); free(W); free(as); free(ws); free(asb); free(wsb); free(rows); free(Y);
}

int main(void)
{
    const int64_t shapes[][3] = {{4, 130, 256}, {5, 33, 200}, {1, 1, 1}, {3, 129, 127}, {2, 300, 384}, {7, 17, 31}};
    for (int kind = 0; kind < 3; ++kind)
        for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
            for (int subset = 0; subset < 2; ++subset)
                one(kind, shapes[i][0], shapes[i][1], shapes[i][2], subset);
    /* empty and degenerate shapes, argument errors */
    double y[4] = {7, 7, 7, 7};
    uint8_t a[4] = {0x38, 0x38, 0x38, 0x38};
    float s[4] = {1, 1, 1, 1};
    int64_t bad_row = 5;
    CHECK(a8w8_oracle_gemm(a, s, a, s, 0, 2, 2, NULL, 0, y) == 0, "M = 0");
    CHECK(a8w8_oracle_gemm(a, s, a, s, 2, 0, 2, NULL, 2, y) == 0, "N = 0");
    CHECK(a8w8_oracle_gemm(a, s, a, s, 2, 2, 0, NULL, 2, y) == 0 && y[0] == 0 && y[3] == 0, "K = 0 gives zeros");
    CHECK(a8w8_oracle_gemm(a, s, a, s, 2, 2, 2, &bad_row, 1, y) == -1, "row out of range");
    CHECK(a8w8_oracle_gemm(a, s, a, s, 2, 2, 2, NULL, 1, y) == -1, "n_rows != M without rows");
    CHECK(a8w8_oracle_gemm(NULL, s, a, s, 2, 2, 2, NULL, 2, y) == -1, "null A");
    CHECK(a8w8_oracle_gemm_mx(a, a, a, a, -1, 2, 2, NULL, 0, y) == -1, "negative M");
    CHECK(a8w8_oracle_gemm_rowwise(a, s, a, s, 2, 2, 2, NULL, 2, NULL) == -1, "null Y");
    for (int c = 0; c < 256; ++c) {
        const double v = a8w8_oracle_e4m3fn_value((uint8_t)c);
        CHECK((c & 0x7F) == 0x7F ? isnan(v) : fabs(v) <= 448.0, "e4m3fn code %d", c);
    }
    if (fails)
        fprintf(stderr, "%d failures\n", fails);
    else
        printf("oracle sanitizer driver: ok\n");
    return fails ? 1 : 0;
}
