/*
 * CPU oracle for Reduced Matrix Multiplication (RMM) -- TEST INFRASTRUCTURE.
 *
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * may build, load or call this file.  The GPU library never links it and
 * shares nothing with it (no headers, helpers or tables).
 *
 * Plain, slow, obviously correct fp64 code written from the definitions in
 * "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction for
 * LLM Inference" (arXiv 2608.13426):
 *   - Sec. 3.2 (definition of RMM_rho): for Y = A B with A n x d, B d x m,
 *     pick an index set I of the contraction axis with |I| = ceil(rho d),
 *     rho in (0, 1], and compute A[:, I] B[I, :];
 *   - Sec. 3.2 (activation-aware dimension selection): score s_j = ||A[:, j]||_2,
 *     I = TopK(s, ceil(rho d)), deterministic;
 *   - Sec. 3.3 (attention): the reduced score product is scaled by
 *     1/sqrt(d_h) with the full head dimension (the caller passes alpha).
 * Readings where the paper is silent (rounding of ceil, tie order, order of
 * I, NaN handling) are stated at each function.
 *
 * Everything is fp64.  Inputs arrive already widened exactly from their
 * storage precision (bf16 or fp32) by the Python wrapper.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * k = ceil(rho * d)  (Sec. 3.2, |I| = ceil(rho d)).
 * Reading: rho is given as a decimal such as 0.7 that binary floating point
 * cannot hold exactly, so rho*d can land a hair above an integer (0.07*100 =
 * 7.000000000000001).  A product within 1e-9 relative of an integer is taken
 * to be that integer before the ceiling.  rho outside (0, 1], NaN, or d < 1
 * give 0 (invalid).  The result is at least 1 and at most d.
 */
int64_t oracle_k(double rho, int64_t d)
{
    if (!(rho > 0.0) || !(rho <= 1.0) || d < 1) return 0;
    double p = rho * (double)d;
    double r = nearbyint(p);
    double tol = 1e-9 * (p > 1.0 ? p : 1.0);
    double kk = (fabs(p - r) <= tol) ? r : ceil(p);
    if (kk < 1.0) kk = 1.0;
    if (kk > (double)d) kk = (double)d;
    return (int64_t)kk;
}

/*
 * s_j = ||A[:, j]||_2 = sqrt(sum_i A[i, j]^2)  (Sec. 3.2 importance score).
 * A is n x d row-major with leading dimension lda.  The sum for each column
 * runs over the rows in ascending order.
 */
void oracle_colnorm(const double *A, int64_t n, int64_t d, int64_t lda, double *s)
{
    for (int64_t j = 0; j < d; ++j) s[j] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double *row = A + i * lda;
        for (int64_t j = 0; j < d; ++j) s[j] += row[j] * row[j];
    }
    for (int64_t j = 0; j < d; ++j) s[j] = sqrt(s[j]);
}

typedef struct {
    double s;
    int64_t j;
} scored_t;

/* Total order used by TopK: larger score first; NaN counts as larger than any
 * number (reading: the paper assumes finite activations); equal scores put
 * the lower index first (reading: the paper only asks for determinism). */
static int by_score_desc_then_index(const void *pa, const void *pb)
{
    const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? -1 : 1;
    if (!an) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    return (a->j < b->j) ? -1 : (a->j > b->j) ? 1 : 0;
}

static int by_index(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * I = TopK(s, k)  (Sec. 3.2): a full sort of all d indices by the total order
 * above, keep the first k, then list them in ascending index order (reading:
 * the paper treats I as a set; ascending order fixes the summation order of
 * the reduced product).  Returns 0 on success, -1 on bad arguments or
 * allocation failure.
 */
int oracle_topk(const double *s, int64_t d, int64_t k, int32_t *idx)
{
    if (d < 1 || k < 1 || k > d) return -1;
    scored_t *v = (scored_t *)malloc((size_t)d * sizeof(scored_t));
    if (!v) return -1;
    for (int64_t j = 0; j < d; ++j) {
        v[j].s = s[j];
        v[j].j = j;
    }
    qsort(v, (size_t)d, sizeof(scored_t), by_score_desc_then_index);
    for (int64_t t = 0; t < k; ++t) idx[t] = (int32_t)v[t].j;
    free(v);
    qsort(idx, (size_t)k, sizeof(int32_t), by_index);
    return 0;
}

typedef struct {
    const double *A;
    int64_t lda;
    const double *B;
    int64_t ldb, m;
    const int32_t *idx;
    int64_t k;
    double alpha;
    const int64_t *rows;
    double *Y;
    int64_t r0, r1;
} product_job_t;

/*
 * Y[r, c] = alpha * sum_{t = 0..k-1} A[i, I_t] * B[I_t, c] with i = rows[r]
 * (the reduced product A[:, I] B[I, :] of Sec. 3.2).  Loop order i, t, c:
 * each output accumulates its k terms in ascending t.
 */
static void *product_rows(void *arg)
{
    product_job_t *jb = (product_job_t *)arg;
    for (int64_t r = jb->r0; r < jb->r1; ++r) {
        int64_t i = jb->rows ? jb->rows[r] : r;
        const double *arow = jb->A + i * jb->lda;
        double *y = jb->Y + r * jb->m;
        for (int64_t c = 0; c < jb->m; ++c) y[c] = 0.0;
        for (int64_t t = 0; t < jb->k; ++t) {
            int64_t j = jb->idx[t];
            double a = arow[j];
            const double *brow = jb->B + j * jb->ldb;
            for (int64_t c = 0; c < jb->m; ++c) y[c] += a * brow[c];
        }
        for (int64_t c = 0; c < jb->m; ++c) y[c] *= jb->alpha;
    }
    return NULL;
}

/*
 * Reduced product over the rows listed in `rows` (nrows entries; NULL means
 * rows 0..nrows-1).  Y is nrows x m, contiguous.  The rows are split over
 * `nthreads` POSIX threads in contiguous ranges; each output is computed by
 * exactly one thread in the order stated above, so the result does not depend
 * on the thread count.  Returns 0 on success.
 */
int oracle_reduced_product(const double *A, int64_t lda, const double *B, int64_t ldb, int64_t m,
                           const int32_t *idx, int64_t k, double alpha, const int64_t *rows,
                           int64_t nrows, double *Y, int nthreads)
{
    if (nrows < 0 || m < 0 || k < 0) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    pthread_t *th = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    product_job_t *jobs = (product_job_t *)malloc((size_t)nthreads * sizeof(product_job_t));
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return -1;
    }
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        product_job_t jb = {A, lda, B, ldb, m, idx, k, alpha, rows, Y, 0, 0};
        jb.r0 = (int64_t)t * per;
        jb.r1 = jb.r0 + per < nrows ? jb.r0 + per : nrows;
        if (jb.r0 > nrows) jb.r0 = nrows;
        jobs[t] = jb;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, product_rows, &jobs[t]) != 0) {
            rc = -1;
            break;
        }
        started = t;
    }
    product_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    if (rc != 0) {
        /* finish whatever the failed threads would have done, serially */
        for (int t = started + 1; t < nthreads; ++t) product_rows(&jobs[t]);
        rc = 0;
    }
    free(th);
    free(jobs);
    return rc;
}
