/*
 * gemm_oracle.c -- the CPU oracle for the dense fp32 matrix product C = A x B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it follows (the pages are web pages on shared-memory tiling):
 *   - "03 CUDA Shared Memory: Tiling, Bank Conflicts, and Reduction",
 *     section "Shared Memory와 Tiling": each output element is the dot product
 *     of one row of A with one column of B, matrices stored row by row in a
 *     single array; tiling only changes where the operands are read from, and
 *     the arithmetic-intensity bookkeeping of the naive and tiled kernels.
 *   - PMPP chapter 5 notes "메모리 계층과 데이터 지역성", sections 5.1 (naive
 *     intensity), 5.3 (traffic per output once tiled), 5.4 (phase loop over
 *     ceil(Width/TILE_WIDTH) phases) and 5.5 (out-of-range tile slots hold
 *     zero and are not loads; only the final store is range checked).
 *   - same first page, section "Bank Conflict": 32 banks of 4-byte words,
 *     n distinct words in one bank serialise into an n-way conflict, equal
 *     words are a broadcast.
 *   - the one-volume PMPP notes, deep-learning chapter: the backward pass
 *     needs the products with a transposed factor, X^T dY and dY W^T, and
 *     runs them on the same tile kernel; op(A), op(B) below.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - general shapes M x K times K x N with row-major leading dimensions
 *     (element (r, c) of a matrix with leading dimension ld sits at r*ld + c);
 *   - the sum runs over k ascending from +0.0 in binary64; every product of
 *     two binary32 values is exact in binary64, so the only rounding is in
 *     the additions;
 *   - alongside C the oracle returns S = sum_k |A_ik| |B_kj|, the scale of
 *     the acceptance bound |C_gpu - C| <= 1e-5 * S.
 *
 * Parity pins (in the CPU tests): exact integer brute force, identity and
 * zero, closed forms, a binary64 library product, linearity, power-of-two
 * scaling, the transpose identity, leading-dimension invariance, transposed
 * operands against explicitly transposed copies, and the pages' printed
 * intensity and bank-conflict numbers.  The per-entry and the
 * traffic/bank functions are pinned the same way; no function here is left
 * "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC -pthread (no -ffast-math: the
 * binary64 additions must happen in the written order).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* ------------------------------------------------------------------------ */
/* One output element: the definition of the product, term by term.         */
/* ------------------------------------------------------------------------ */

/* c = sum_{k=0}^{K-1} A[i][k] * B[k][j]   and   s = sum_k |A[i][k] * B[k][j]|,
 * where element (i, k) of the left factor is A[i*a_rs + k*a_cs] and element
 * (k, j) of the right factor is B[k*b_rs + j*b_cs].  A row-major matrix with
 * leading dimension ld has (row stride, column stride) = (ld, 1); its
 * transpose, read in place, has (1, ld). */
static void dot_entry(int64_t K, const float *A, int64_t a_rs, int64_t a_cs,
                      const float *B, int64_t b_rs, int64_t b_cs,
                      int64_t i, int64_t j, double *c, double *s)
{
    double acc = 0.0;
    double mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double prod = (double)A[i * a_rs + k * a_cs] * (double)B[k * b_rs + j * b_cs];
        acc += prod;
        mag += fabs(prod);
    }
    *c = acc;
    *s = mag;
}

/* Strides of op(X) for a stored row-major X with leading dimension ld:
 * op 0 uses X as stored, op 1 uses its transpose. */
static void op_strides(int op, int64_t ld, int64_t *rs, int64_t *cs)
{
    if (op == 0) { *rs = ld; *cs = 1; }
    else         { *rs = 1;  *cs = ld; }
}

/* ------------------------------------------------------------------------ */
/* Full product.  Rows are handed out to worker threads in contiguous       */
/* blocks; each element is computed by exactly one thread with the same     */
/* per-element code, so the result does not depend on the thread count.     */
/* ------------------------------------------------------------------------ */

struct rows_job {
    int64_t row_begin, row_end, N, K;
    const float *A; int64_t a_rs, a_cs;
    const float *B; int64_t b_rs, b_cs;
    double *C; int64_t ldc;
    double *S; int64_t lds;
};

static void *rows_worker(void *arg)
{
    const struct rows_job *job = (const struct rows_job *)arg;
    for (int64_t i = job->row_begin; i < job->row_end; ++i) {
        for (int64_t j = 0; j < job->N; ++j) {
            double c, s;
            dot_entry(job->K, job->A, job->a_rs, job->a_cs, job->B, job->b_rs, job->b_cs,
                      i, j, &c, &s);
            job->C[i * job->ldc + j] = c;
            if (job->S)
                job->S[i * job->lds + j] = s;
        }
    }
    return NULL;
}

/* C (binary64, leading dimension ldc) = op(A) x op(B); S (optional, may be
 * NULL, leading dimension lds) = sum of |products|.  op_a = 0: A is stored
 * M x K (lda >= K); op_a = 1: A is stored K x M (lda >= M) and op(A) is its
 * transpose.  op_b = 0: B is stored K x N (ldb >= N); op_b = 1: B is stored
 * N x K (ldb >= K).  Rows [row_begin, row_end) of the product only, so a
 * caller can time or check a band of rows.  threads <= 1 runs on the
 * calling thread. */
int oracle_gemm_op_rows(int op_a, int op_b, int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda, const float *B, int64_t ldb,
                        double *C, int64_t ldc, double *S, int64_t lds,
                        int64_t row_begin, int64_t row_end, int threads)
{
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || row_begin < 0 || row_end > M || row_begin > row_end)
        return ORACLE_BAD_ARG;
    int64_t a_cols = op_a == 0 ? K : M, b_cols = op_b == 0 ? N : K;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if (S && lds < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if ((row_end > row_begin && N > 0) && (!C || (K > 0 && (!A || !B))))
        return ORACLE_BAD_ARG;
    int64_t a_rs, a_cs, b_rs, b_cs;
    op_strides(op_a, lda, &a_rs, &a_cs);
    op_strides(op_b, ldb, &b_rs, &b_cs);

    int64_t rows = row_end - row_begin;
    if (threads < 1)
        threads = 1;
    if (threads > rows)
        threads = rows > 0 ? (int)rows : 1;

    struct rows_job *jobs = (struct rows_job *)calloc((size_t)threads, sizeof *jobs);
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof *tids);
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return ORACLE_BAD_ARG;
    }
    int64_t per = rows / threads, extra = rows % threads, r = row_begin;
    for (int t = 0; t < threads; ++t) {
        int64_t take = per + (t < extra ? 1 : 0);
        jobs[t] = (struct rows_job){r, r + take, N, K, A, a_rs, a_cs, B, b_rs, b_cs, C, ldc, S, lds};
        r += take;
    }
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tids[t], NULL, rows_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    rows_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    for (int t = started + 1; t < threads; ++t) /* threads that failed to start */
        rows_worker(&jobs[t]);
    free(jobs);
    free(tids);
    return ORACLE_OK;
}

/* The plain product C = A x B (both as stored), rows [row_begin, row_end). */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     double *C, int64_t ldc, double *S, int64_t lds,
                     int64_t row_begin, int64_t row_end, int threads)
{
    return oracle_gemm_op_rows(0, 0, M, N, K, A, lda, B, ldb, C, ldc, S, lds,
                               row_begin, row_end, threads);
}

int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda, const float *B, int64_t ldb,
                double *C, int64_t ldc, double *S, int64_t lds, int threads)
{
    return oracle_gemm_rows(M, N, K, A, lda, B, ldb, C, ldc, S, lds, 0, M, threads);
}

/* Selected entries only: out_c[t], out_s[t] for the pair (ii[t], jj[t]) of
 * op(A) x op(B) (op flags as in oracle_gemm_op_rows).  Used where the full
 * product is too large to compute on the host. */
int oracle_gemm_op_entries(int op_a, int op_b, int64_t M, int64_t N, int64_t K,
                           const float *A, int64_t lda, const float *B, int64_t ldb,
                           int64_t count, const int64_t *ii, const int64_t *jj,
                           double *out_c, double *out_s)
{
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_BAD_ARG;
    int64_t a_cols = op_a == 0 ? K : M, b_cols = op_b == 0 ? N : K;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1))
        return ORACLE_BAD_ARG;
    int64_t a_rs, a_cs, b_rs, b_cs;
    op_strides(op_a, lda, &a_rs, &a_cs);
    op_strides(op_b, ldb, &b_rs, &b_cs);
    for (int64_t t = 0; t < count; ++t) {
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return ORACLE_BAD_ARG;
        double c, s;
        dot_entry(K, A, a_rs, a_cs, B, b_rs, b_cs, ii[t], jj[t], &c, &s);
        out_c[t] = c;
        if (out_s)
            out_s[t] = s;
    }
    return ORACLE_OK;
}

int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda, const float *B, int64_t ldb,
                        int64_t count, const int64_t *ii, const int64_t *jj,
                        double *out_c, double *out_s)
{
    return oracle_gemm_op_entries(0, 0, M, N, K, A, lda, B, ldb, count, ii, jj, out_c, out_s);
}

/* ------------------------------------------------------------------------ */
/* Global-traffic bookkeeping of the tiled phase loop, by brute force.      */
/* ------------------------------------------------------------------------ */

/* Walks every workgroup tile (BM rows x BN columns of C) and every phase of
 * BK along k, exactly as the tiled kernel's loop does, and counts for each
 * staged tile slot whether it is a real global read or a zero "ghost" slot.
 * The naive one-thread-per-output kernel is the case BM = BN = BK = 1: each
 * "tile" is a single output, and every k step reads one A and one B element.
 *
 *   out[0] = A elements read from global memory
 *   out[1] = B elements read from global memory
 *   out[2] = A ghost slots (zero filled, not read)
 *   out[3] = B ghost slots
 *   out[4] = multiply-adds issued (ghost ones included)
 *   out[5] = useful multiply-adds (both operands in range)
 *   out[6] = number of workgroup tiles
 *   out[7] = number of phases per tile
 */
int oracle_tiled_traffic(int64_t M, int64_t N, int64_t K,
                         int64_t BM, int64_t BN, int64_t BK, int64_t *out)
{
    if (M < 0 || N < 0 || K < 0 || BM < 1 || BN < 1 || BK < 1 || !out)
        return ORACLE_BAD_ARG;
    for (int q = 0; q < 8; ++q)
        out[q] = 0;
    int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int64_t phases = (K + BK - 1) / BK;
    out[6] = tiles_m * tiles_n;
    out[7] = phases;
    for (int64_t tm = 0; tm < tiles_m; ++tm) {
        for (int64_t tn = 0; tn < tiles_n; ++tn) {
            for (int64_t p = 0; p < phases; ++p) {
                /* A tile: rows tm*BM .. +BM, columns (k) p*BK .. +BK */
                for (int64_t r = 0; r < BM; ++r)
                    for (int64_t c = 0; c < BK; ++c) {
                        int64_t row = tm * BM + r, k = p * BK + c;
                        if (row < M && k < K) out[0]++; else out[2]++;
                    }
                /* B tile: rows (k) p*BK .. +BK, columns tn*BN .. +BN */
                for (int64_t r = 0; r < BK; ++r)
                    for (int64_t c = 0; c < BN; ++c) {
                        int64_t k = p * BK + r, col = tn * BN + c;
                        if (k < K && col < N) out[1]++; else out[3]++;
                    }
                /* inner products over the staged tiles */
                for (int64_t r = 0; r < BM; ++r)
                    for (int64_t c = 0; c < BN; ++c)
                        for (int64_t kk = 0; kk < BK; ++kk) {
                            out[4]++;
                            int64_t row = tm * BM + r, col = tn * BN + c, k = p * BK + kk;
                            if (row < M && col < N && k < K)
                                out[5]++;
                        }
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Shared-memory bank model, by brute force.                                 */
/* ------------------------------------------------------------------------ */

/* Given the 4-byte word address each lane touches in one access, returns the
 * conflict degree: the largest number of DISTINCT words that fall into one
 * bank (word w lives in bank w mod banks).  Equal words are one broadcast and
 * count once.  A degree of 1 means the access is conflict free. */
int64_t oracle_bank_conflict_degree(int64_t lanes, const int64_t *word_addr,
                                    int64_t banks)
{
    if (lanes < 0 || banks < 1 || (lanes > 0 && !word_addr))
        return -1;
    int64_t worst = lanes > 0 ? 1 : 0;
    for (int64_t b = 0; b < banks; ++b) {
        int64_t distinct = 0;
        for (int64_t l = 0; l < lanes; ++l) {
            int64_t w = word_addr[l];
            if (((w % banks) + banks) % banks != b)
                continue;
            int seen = 0;
            for (int64_t e = 0; e < l; ++e)
                if (word_addr[e] == w) { seen = 1; break; }
            if (!seen)
                distinct++;
        }
        if (distinct > worst)
            worst = distinct;
    }
    return worst;
}
