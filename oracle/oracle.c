/*
 * CPU oracle for C = A * B on CSR matrices. TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may call this file. The GPU library never links, loads or calls it, and
 * it shares no code, header or table with the GPU library.
 *
 * What it computes is the plain definition of the sparse product, written as
 * Gustavson's row-by-row method (gMAGNUS page, Section II-B, Eq. 1 and
 * Algorithm 1): row i of C is the sum over the stored A[i,k] of A[i,k] times
 * row k of B, and the row is written with its columns in ascending order
 * (the "SortAndWrite" step of Algorithm 1). The per-row count of
 * intermediate products is u(i) = sum over k in row i of A of nnz(B[k,:])
 * (SparseDitto page, Section 3, Eq. 1).
 *
 * Per row the oracle
 *   1. emits every product (j, a*b) in storage order: A's entries of the row
 *      in CSR order, and for each, B's entries of row k in CSR order; a*b is
 *      one IEEE-754 double multiply;
 *   2. orders the products by column, breaking ties by emission order;
 *   3. sums each run of equal columns in emission order in long double
 *      (x86-64 80-bit, 64-bit significand) and rounds the sum once to
 *      double; it also returns the run's sum of |a*b| in double for the
 *      error bound |c_gpu - c_ref| <= 1e-12 * sum|a*b|;
 *   4. keeps every reachable column, including sums that cancel to zero.
 *
 * Rows are spread over POSIX threads, taken dynamically in small blocks.
 * Nothing here is tuned; it is meant to be read against the definition.
 */
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if LDBL_MANT_DIG < 64
#error "the oracle accumulates in an extended long double (64-bit significand)"
#endif

typedef struct {
    int64_t nrows, ncols;
    const int64_t* rowptr;
    const int32_t* col;
    const double* val;
} ocsr;

typedef struct {
    int64_t nsel;     /* number of rows computed                        */
    int64_t nnz;      /* total entries over those rows                  */
    int64_t* rowptr;  /* nsel+1 offsets into col/val/abssum             */
    int32_t* col;     /* ascending within each row                       */
    double* val;      /* long-double sum rounded once to double          */
    double* abssum;   /* sum of |a*b| over the entry's products          */
    int64_t* u;       /* intermediate products per computed row          */
} oracle_result;

/* one emitted product */
typedef struct {
    int32_t col;
    int64_t seq;
    double prod;
} oprod;

static int cmp_prod(const void* x, const void* y) {
    const oprod* a = (const oprod*)x;
    const oprod* b = (const oprod*)y;
    if (a->col != b->col) return a->col < b->col ? -1 : 1;
    if (a->seq != b->seq) return a->seq < b->seq ? -1 : 1;
    return 0;
}

/* u(i) for every row of A (exact integer count of intermediate products). */
int oracle_row_products(int64_t an, const int64_t* arp, const int32_t* acol,
                        const int64_t* brp, int64_t* u_out) {
    for (int64_t i = 0; i < an; ++i) {
        int64_t s = 0;
        for (int64_t q = arp[i]; q < arp[i + 1]; ++q) {
            int32_t k = acol[q];
            s += brp[k + 1] - brp[k];
        }
        u_out[i] = s;
    }
    return 0;
}

/* Per-row result kept until all rows are done, then concatenated. */
typedef struct {
    int64_t n;
    int32_t* col;
    double* val;
    double* abssum;
    int64_t u;
} orow;

typedef struct {
    const ocsr* A;
    const ocsr* B;
    const int64_t* rows;
    int64_t nsel;
    orow* out;
    int64_t next; /* next unclaimed index into rows */
    pthread_mutex_t lock;
    int failed;
} ojob;

static int compute_row(const ocsr* A, const ocsr* B, int64_t i, orow* r) {
    int64_t u = 0;
    for (int64_t q = A->rowptr[i]; q < A->rowptr[i + 1]; ++q) {
        int32_t k = A->col[q];
        u += B->rowptr[k + 1] - B->rowptr[k];
    }
    r->u = u;
    r->n = 0;
    r->col = NULL;
    r->val = NULL;
    r->abssum = NULL;
    if (u == 0) return 0;

    /* 1. emit products in storage order */
    oprod* p = (oprod*)malloc((size_t)u * sizeof(oprod));
    if (!p) return -1;
    int64_t t = 0;
    for (int64_t q = A->rowptr[i]; q < A->rowptr[i + 1]; ++q) {
        int32_t k = A->col[q];
        double a = A->val[q];
        for (int64_t e = B->rowptr[k]; e < B->rowptr[k + 1]; ++e) {
            p[t].col = B->col[e];
            p[t].seq = t;
            p[t].prod = a * B->val[e];
            ++t;
        }
    }
    /* 2. order by column, ties by emission order */
    qsort(p, (size_t)u, sizeof(oprod), cmp_prod);

    /* 3. count the runs, then sum each run */
    int64_t nruns = 0;
    for (int64_t x = 0; x < u; ++x)
        if (x == 0 || p[x].col != p[x - 1].col) ++nruns;
    r->col = (int32_t*)malloc((size_t)nruns * sizeof(int32_t));
    r->val = (double*)malloc((size_t)nruns * sizeof(double));
    r->abssum = (double*)malloc((size_t)nruns * sizeof(double));
    if (!r->col || !r->val || !r->abssum) {
        free(p);
        return -1;
    }
    int64_t o = 0;
    int64_t x = 0;
    while (x < u) {
        int32_t c = p[x].col;
        long double s = 0.0L;
        long double sa = 0.0L;
        while (x < u && p[x].col == c) {
            s += (long double)p[x].prod;
            sa += (long double)(p[x].prod < 0 ? -p[x].prod : p[x].prod);
            ++x;
        }
        r->col[o] = c;
        r->val[o] = (double)s;
        r->abssum[o] = (double)sa;
        ++o;
    }
    r->n = nruns;
    free(p);
    return 0;
}

static void* worker(void* arg) {
    ojob* job = (ojob*)arg;
    const int64_t block = 16;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int64_t s = job->next;
        job->next += block;
        int failed = job->failed;
        pthread_mutex_unlock(&job->lock);
        if (s >= job->nsel || failed) break;
        int64_t e = s + block < job->nsel ? s + block : job->nsel;
        for (int64_t x = s; x < e; ++x) {
            if (compute_row(job->A, job->B, job->rows[x], &job->out[x]) != 0) {
                pthread_mutex_lock(&job->lock);
                job->failed = 1;
                pthread_mutex_unlock(&job->lock);
                return NULL;
            }
        }
    }
    return NULL;
}

void oracle_free(oracle_result* res) {
    if (!res) return;
    free(res->rowptr);
    free(res->col);
    free(res->val);
    free(res->abssum);
    free(res->u);
    memset(res, 0, sizeof(*res));
}

/*
 * Compute the rows listed in `rows` (any order, repeats allowed) of A*B.
 * Pointers are host pointers. Returns 0 on success, -1 on a bad argument,
 * -2 when memory runs out. On success the caller owns `res` and releases it
 * with oracle_free().
 */
int oracle_spgemm_rows(int64_t an, int64_t am, const int64_t* arp, const int32_t* acol,
                       const double* aval, int64_t bn, int64_t bm, const int64_t* brp,
                       const int32_t* bcol, const double* bval, const int64_t* rows,
                       int64_t nsel, int nthreads, oracle_result* res) {
    if (!res || am != bn || nsel < 0 || an < 0 || bm < 0) return -1;
    memset(res, 0, sizeof(*res));
    for (int64_t x = 0; x < nsel; ++x)
        if (rows[x] < 0 || rows[x] >= an) return -1;
    ocsr A = {an, am, arp, acol, aval};
    ocsr B = {bn, bm, brp, bcol, bval};
    orow* out = (orow*)calloc((size_t)(nsel > 0 ? nsel : 1), sizeof(orow));
    if (!out) return -2;

    ojob job;
    job.A = &A;
    job.B = &B;
    job.rows = rows;
    job.nsel = nsel;
    job.out = out;
    job.next = 0;
    job.failed = 0;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &job) != 0) break;
        ++started;
    }
    if (started == 0) worker(&job);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&job.lock);

    int rc = job.failed ? -2 : 0;
    int64_t nnz = 0;
    for (int64_t x = 0; x < nsel && rc == 0; ++x) nnz += out[x].n;
    if (rc == 0) {
        res->nsel = nsel;
        res->nnz = nnz;
        res->rowptr = (int64_t*)malloc((size_t)(nsel + 1) * sizeof(int64_t));
        res->u = (int64_t*)malloc((size_t)(nsel > 0 ? nsel : 1) * sizeof(int64_t));
        res->col = (int32_t*)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int32_t));
        res->val = (double*)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(double));
        res->abssum = (double*)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(double));
        if (!res->rowptr || !res->u || !res->col || !res->val || !res->abssum) rc = -2;
    }
    if (rc == 0) {
        int64_t o = 0;
        res->rowptr[0] = 0;
        for (int64_t x = 0; x < nsel; ++x) {
            if (out[x].n) {
                memcpy(res->col + o, out[x].col, (size_t)out[x].n * sizeof(int32_t));
                memcpy(res->val + o, out[x].val, (size_t)out[x].n * sizeof(double));
                memcpy(res->abssum + o, out[x].abssum, (size_t)out[x].n * sizeof(double));
            }
            o += out[x].n;
            res->rowptr[x + 1] = o;
            res->u[x] = out[x].u;
        }
    }
    for (int64_t x = 0; x < nsel; ++x) {
        free(out[x].col);
        free(out[x].val);
        free(out[x].abssum);
    }
    free(out);
    if (rc != 0) oracle_free(res);
    return rc;
}
