/*
 * Driver for the C oracle (oracle/rmm_oracle.c) built with sanitizers
 * (tests/test_sanitizers.py): AddressSanitizer + UndefinedBehaviorSanitizer
 * in one build, ThreadSanitizer in another.  It runs every exported function
 * on small seeded inputs and on the edge cases (k = 1, k = d, ties, NaN
 * scores, zero rows or columns, more threads than rows) and checks results
 * that hold by construction: the kept set is ascending and holds k distinct
 * indices, the multi-threaded product equals the single-threaded one bit for
 * bit, and the product over every index equals the plain triple loop.
 * Prints "ok" and exits 0; a sanitizer report ends it with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_k(double rho, int64_t d);
void oracle_colnorm(const double *A, int64_t n, int64_t d, int64_t lda, double *s);
int oracle_topk(const double *s, int64_t d, int64_t k, int32_t *idx);
int oracle_reduced_product(const double *A, int64_t lda, const double *B, int64_t ldb, int64_t m,
                           const int32_t *idx, int64_t k, double alpha, const int64_t *rows, int64_t nrows,
                           double *Y, int nthreads);

static int fails = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                                      \
        }                                                                 \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) /* splitmix64 -> [-1, 1) */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static void check_set(const int32_t *idx, int64_t k, int64_t d)
{
    for (int64_t t = 0; t < k; ++t) {
        CHECK(idx[t] >= 0 && idx[t] < d);
        if (t) CHECK(idx[t - 1] < idx[t]);
    }
}

static void one_case(int64_t n, int64_t d, int64_t m, double rho, int nthreads)
{
    const int64_t lda = d + 3, ldb = m + 1;
    double *A = malloc(sizeof(double) * (size_t)(n * lda + 1));
    double *B = malloc(sizeof(double) * (size_t)(d * ldb + 1));
    double *s = malloc(sizeof(double) * (size_t)d);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)d);
    double *Y1 = malloc(sizeof(double) * (size_t)(n * m + 1));
    double *Yt = malloc(sizeof(double) * (size_t)(n * m + 1));
    for (int64_t i = 0; i < n * lda; ++i) A[i] = uniform();
    for (int64_t i = 0; i < d * ldb; ++i) B[i] = uniform();
    if (d > 3) { /* ties: two equal columns, and a zero column */
        for (int64_t i = 0; i < n; ++i) {
            A[i * lda + 1] = A[i * lda + 2];
            A[i * lda + 3] = 0.0;
        }
    }
    const int64_t k = oracle_k(rho, d);
    CHECK(k >= 1 && k <= d);
    oracle_colnorm(A, n, d, lda, s);
    CHECK(oracle_topk(s, d, k, idx) == 0);
    check_set(idx, k, d);
    CHECK(oracle_reduced_product(A, lda, B, ldb, m, idx, k, 0.5, NULL, n, Y1, 1) == 0);
    CHECK(oracle_reduced_product(A, lda, B, ldb, m, idx, k, 0.5, NULL, n, Yt, nthreads) == 0);
    CHECK(memcmp(Y1, Yt, sizeof(double) * (size_t)(n * m)) == 0);
    /* every index kept: the plain product */
    for (int64_t j = 0; j < d; ++j) idx[j] = (int32_t)j;
    CHECK(oracle_reduced_product(A, lda, B, ldb, m, idx, d, 1.0, NULL, n, Yt, nthreads) == 0);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t c = 0; c < m; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < d; ++j) acc += A[i * lda + j] * B[j * ldb + c];
            CHECK(Yt[i * m + c] == acc);
        }
    /* a subset of rows, in a shuffled order */
    if (n > 2) {
        int64_t rows[3] = {n - 1, 0, n / 2};
        CHECK(oracle_reduced_product(A, lda, B, ldb, m, idx, d, 1.0, rows, 3, Y1, nthreads) == 0);
        for (int r = 0; r < 3; ++r)
            for (int64_t c = 0; c < m; ++c) CHECK(Y1[r * m + c] == Yt[rows[r] * m + c]);
    }
    free(A);
    free(B);
    free(s);
    free(idx);
    free(Y1);
    free(Yt);
}

int main(void)
{
    /* k = ceil(rho d) and its invalid arguments */
    CHECK(oracle_k(0.8, 4096) == 3277);
    CHECK(oracle_k(0.07, 100) == 7);
    CHECK(oracle_k(0.0, 10) == 0 && oracle_k(1.5, 10) == 0 && oracle_k(NAN, 10) == 0 && oracle_k(0.5, 0) == 0);
    CHECK(oracle_k(1e-9, 5) == 1);

    one_case(1, 1, 1, 1.0, 1);
    one_case(7, 9, 3, 0.2, 4);
    one_case(33, 65, 72, 0.999, 8);
    one_case(5, 37, 13, 0.5, 16); /* more threads than rows */
    one_case(64, 300, 24, 0.01, 3);

    /* TopK: NaN above every number, ties to the lower index, bad arguments */
    double s[6] = {1.0, NAN, 3.0, 3.0, -INFINITY, 0.0};
    int32_t idx[6];
    CHECK(oracle_topk(s, 6, 2, idx) == 0 && idx[0] == 1 && idx[1] == 2);
    CHECK(oracle_topk(s, 6, 3, idx) == 0 && idx[0] == 1 && idx[1] == 2 && idx[2] == 3);
    CHECK(oracle_topk(s, 6, 6, idx) == 0);
    check_set(idx, 6, 6);
    CHECK(oracle_topk(s, 6, 0, idx) == -1 && oracle_topk(s, 6, 7, idx) == -1 && oracle_topk(s, 0, 1, idx) == -1);
    /* empty products */
    double y = 7.0;
    CHECK(oracle_reduced_product(s, 1, s, 1, 0, idx, 1, 1.0, NULL, 1, &y, 2) == 0);
    CHECK(oracle_reduced_product(s, 1, s, 1, 1, idx, 0, 1.0, NULL, 0, &y, 2) == 0);
    CHECK(oracle_reduced_product(s, 1, s, 1, 1, idx, 1, 1.0, NULL, -1, &y, 2) == -1);

    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
