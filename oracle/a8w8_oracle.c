/*
 * a8w8_oracle.c -- plain fp64 CPU reference for the a8w8 block-scale GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (the plain definition, written out):
 *
 *   Ad[m,k] = e4m3fn(A[m,k]) * a_scale[m, k/128]
 *   Wd[n,k] = e4m3fn(W[n,k]) * w_scale[n/128, k/128]
 *   Y[m,n]  = sum_k Ad[m,k] * Wd[n,k]            (fp64, k ascending, not rounded)
 *
 * By distributivity this equals sum over 128-wide K blocks kb of
 * (A_fp8 . W_fp8^T)_kb * a_scale[m,kb] * w_scale[n/128,kb], the block-scale
 * GEMM "gemm_a8w8_blockscale" that the pages tune ("Retune gfx942 Qwen3.8-27B
 * a8w8 blockscale decode rows for cold weights", Kernel section) for
 * checkpoints quantised with 128x128 weight blocks ("Why aiter#5069's measured
 * -25% kernel win moved serving throughput by 0.0%", the unreachable-half
 * paragraph).  The pages name the operation but print no formula; the 1x128
 * activation groups and 128x128 weight blocks with fp32 scales are this
 * project's reading.
 *
 * Layouts (row-major): A uint8 [M,K]; a_scale float [M, ceil(K/128)];
 * W uint8 [N,K]; w_scale float [ceil(N/128), ceil(K/128)]; Y double
 * [n_rows, N] for the requested rows of Y (all M rows when rows == NULL).
 * K need not be a multiple of 128 here: the last group is simply short.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Value of one OCP 8-bit floating point E4M3 byte ("e4m3fn"): sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 holds the
 * subnormals (mantissa/8) * 2^-6; S.1111.111 is NaN; there are no infinities,
 * so the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double a8w8_oracle_e4m3fn_value(uint8_t code)
{
    int sign = code >> 7;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double mag;
    if (expo == 0xF && mant == 0x7)
        return NAN;
    if (expo == 0)
        mag = ldexp((double)mant, -9);                 /* (mant/8) * 2^(1-7) */
    else
        mag = ldexp((double)(8 + mant), expo - 10);    /* (1 + mant/8) * 2^(expo-7) */
    return sign ? -mag : mag;
}

int a8w8_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Y[r, n] for r < n_rows (row m = rows[r], or m = r when rows == NULL), n < N.
 * Returns 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
int a8w8_oracle_gemm(const uint8_t *A, const float *a_scale,
                     const uint8_t *W, const float *w_scale,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows, double *Y)
{
    const int64_t G = 128;
    int64_t KB, r, nb, NB;
    double table[256];
    double *Ad;
    int bad = 0;

    if (M < 0 || N < 0 || K < 0 || n_rows < 0)
        return -1;
    if (rows == NULL && n_rows != M)
        return -1;
    if (n_rows == 0 || N == 0)
        return 0;
    if (K == 0) {
        memset(Y, 0, (size_t)(n_rows * N) * sizeof(double));
        return 0;
    }
    if (!A || !a_scale || !W || !w_scale || !Y)
        return -1;
    for (r = 0; r < n_rows; ++r) {
        int64_t m = rows ? rows[r] : r;
        if (m < 0 || m >= M)
            return -1;
    }

    for (int c = 0; c < 256; ++c)
        table[c] = a8w8_oracle_e4m3fn_value((uint8_t)c);

    KB = (K + G - 1) / G;
    NB = (N + G - 1) / G;

    /* Dequantised activation rows (fp64; each value dec(q) * scale is exact in fp64). */
    Ad = (double *)malloc((size_t)(n_rows * K) * sizeof(double));
    if (!Ad)
        return -2;
    for (r = 0; r < n_rows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t k = 0; k < K; ++k)
            Ad[r * K + k] = table[A[m * K + k]] * (double)a_scale[m * KB + k / G];
    }

    /* One 128-row block of W at a time: dequantise it, then take the dots. */
#pragma omp parallel for schedule(dynamic, 1)
    for (nb = 0; nb < NB; ++nb) {
        int64_t n0 = nb * G;
        int64_t rows_here = (N - n0 < G) ? (N - n0) : G;
        double *Wd = (double *)malloc((size_t)(rows_here * K) * sizeof(double));
        if (!Wd) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t i = 0; i < rows_here; ++i)
            for (int64_t k = 0; k < K; ++k)
                Wd[i * K + k] = table[W[(n0 + i) * K + k]] * (double)w_scale[nb * KB + k / G];
        for (int64_t rr = 0; rr < n_rows; ++rr) {
            const double *a = Ad + rr * K;
            for (int64_t i = 0; i < rows_here; ++i) {
                const double *w = Wd + i * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += a[k] * w[k];
                Y[rr * N + n0 + i] = acc;
            }
        }
        free(Wd);
    }
    free(Ad);
    return bad ? -2 : 0;
}

/*
 * MX-scaled variant: the "32x32" weight-scale blocks of the mxfp8 GEMMs on the
 * gfx1250 BF16 and MX32 tuned-rows page (ROCm/aiter #7247, Motivation and
 * Technical Details).  That page gives the block shape of the weight scales
 * and the "mxfp8" element type but no formula; the reading here follows the
 * OCP Microscaling (MX) format: every scale is one E8M0 byte (an unsigned
 * power-of-two exponent with bias 127, 0xFF = NaN), activations carry one
 * scale per row per 32-wide K group and weights one per 32 x 32 block.
 *
 *   Ad[m,k] = e4m3fn(A[m,k]) * e8m0(a_scale[m, k/32])
 *   Wd[n,k] = e4m3fn(W[n,k]) * e8m0(w_scale[n/32, k/32])
 *   Y[m,n]  = sum_k Ad[m,k] * Wd[n,k]            (fp64, k ascending, not rounded)
 *
 * Layouts (row-major): A uint8 [M,K]; a_scale uint8 [M, ceil(K/32)];
 * W uint8 [N,K]; w_scale uint8 [ceil(N/32), ceil(K/32)]; Y double [n_rows, N].
 */
double a8w8_oracle_e8m0_value(uint8_t code)
{
    if (code == 0xFF)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

int a8w8_oracle_gemm_mx(const uint8_t *A, const uint8_t *a_scale,
                        const uint8_t *W, const uint8_t *w_scale,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t *rows, int64_t n_rows, double *Y)
{
    const int64_t G = 32;
    int64_t KG, r, nb, NB;
    double table[256], scale[256];
    double *Ad;
    int bad = 0;

    if (M < 0 || N < 0 || K < 0 || n_rows < 0)
        return -1;
    if (rows == NULL && n_rows != M)
        return -1;
    if (n_rows == 0 || N == 0)
        return 0;
    if (K == 0) {
        memset(Y, 0, (size_t)(n_rows * N) * sizeof(double));
        return 0;
    }
    if (!A || !a_scale || !W || !w_scale || !Y)
        return -1;
    for (r = 0; r < n_rows; ++r) {
        int64_t m = rows ? rows[r] : r;
        if (m < 0 || m >= M)
            return -1;
    }

    for (int c = 0; c < 256; ++c) {
        table[c] = a8w8_oracle_e4m3fn_value((uint8_t)c);
        scale[c] = a8w8_oracle_e8m0_value((uint8_t)c);
    }

    KG = (K + G - 1) / G;
    NB = (N + G - 1) / G;

    /* Dequantised activation rows (each dec(q) * 2^e is exact in fp64). */
    Ad = (double *)malloc((size_t)(n_rows * K) * sizeof(double));
    if (!Ad)
        return -2;
    for (r = 0; r < n_rows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t k = 0; k < K; ++k)
            Ad[r * K + k] = table[A[m * K + k]] * scale[a_scale[m * KG + k / G]];
    }

    /* One 32-row block of W at a time: dequantise it, then take the dots. */
#pragma omp parallel for schedule(dynamic, 1)
    for (nb = 0; nb < NB; ++nb) {
        int64_t n0 = nb * G;
        int64_t rows_here = (N - n0 < G) ? (N - n0) : G;
        double *Wd = (double *)malloc((size_t)(rows_here * K) * sizeof(double));
        if (!Wd) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t i = 0; i < rows_here; ++i)
            for (int64_t k = 0; k < K; ++k)
                Wd[i * K + k] = table[W[(n0 + i) * K + k]] * scale[w_scale[nb * KG + k / G]];
        for (int64_t rr = 0; rr < n_rows; ++rr) {
            const double *a = Ad + rr * K;
            for (int64_t i = 0; i < rows_here; ++i) {
                const double *w = Wd + i * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += a[k] * w[k];
                Y[rr * N + n0 + i] = acc;
            }
        }
        free(Wd);
    }
    free(Ad);
    return bad ? -2 : 0;
}

/*
 * Row-wise ("per-token") variant: one fp32 scale per activation row and one
 * per weight row (output channel), the non-block-scale a8w8 path that the
 * "Why aiter#5069's measured -25% kernel win moved serving throughput by
 * 0.0%" page describes as fed by a per-token fp8 setting (unreachable for its
 * block-quantised checkpoint).  The pages give no formula; the reading here
 * is the plain row-wise scaled product:
 *
 *   Y[m,n] = a_scale[m] * w_scale[n] * sum_k e4m3fn(A[m,k]) * e4m3fn(W[n,k])
 *
 * (fp64; the sum over k ascending, then the two scales, not rounded).
 * Layouts: A uint8 [M,K]; a_scale float [M]; W uint8 [N,K]; w_scale float [N];
 * Y double [n_rows, N] for the requested rows (all M when rows == NULL).
 */
int a8w8_oracle_gemm_rowwise(const uint8_t *A, const float *a_scale,
                             const uint8_t *W, const float *w_scale,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t *rows, int64_t n_rows, double *Y)
{
    double table[256];
    int64_t r, n;

    if (M < 0 || N < 0 || K < 0 || n_rows < 0)
        return -1;
    if (rows == NULL && n_rows != M)
        return -1;
    if (n_rows == 0 || N == 0)
        return 0;
    if (!A || !a_scale || !W || !w_scale || !Y)
        return -1;
    for (r = 0; r < n_rows; ++r) {
        int64_t m = rows ? rows[r] : r;
        if (m < 0 || m >= M)
            return -1;
    }
    for (int c = 0; c < 256; ++c)
        table[c] = a8w8_oracle_e4m3fn_value((uint8_t)c);

#pragma omp parallel for schedule(dynamic, 16)
    for (n = 0; n < N; ++n) {
        for (int64_t rr = 0; rr < n_rows; ++rr) {
            int64_t m = rows ? rows[rr] : rr;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += table[A[m * K + k]] * table[W[n * K + k]];
            Y[rr * N + n] = acc * (double)a_scale[m] * (double)w_scale[n];
        }
    }
    return 0;
}
