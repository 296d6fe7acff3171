/*
 * gemm16_oracle.c -- the CPU oracle for the mixed-precision product: both
 * factors in a 16-bit format (bfloat16 or IEEE binary16), the result in
 * binary32.
 *
 * TEST INFRASTRUCTURE ONLY, like gemm_oracle.c: nothing in the product path
 * may include, link, load or call it.
 *
 * What it follows:
 *   - the one-volume PMPP notes ("PMPP 단권화"), deep-learning chapter: a
 *     fully connected layer is a matrix product ("FC Layer = GEMM"), run on
 *     matrix units that take FP16 or BF16 inputs and accumulate in FP32; in
 *     "Mixed Precision", BF16 has the exponent range of FP32, while FP16's
 *     narrow range is what loss scaling works around;
 *   - same chapter: the backward pass needs the products with a transposed
 *     factor (X^T dY, dY W^T); op(A), op(B) below, as in gemm_oracle.c;
 *   - same notes, reduction chapter, numerical remarks: sums of 16-bit values
 *     risk overflow, hence an FP32 accumulator;
 *   - the two formats as they are defined.  binary16 (IEEE 754-2008): sign
 *     bit, 5 exponent bits with bias 15, 10 fraction bits; exponent field 0
 *     holds zero and the subnormals f 2^-24, field 31 infinities and NaNs.
 *     bfloat16: sign bit, 8 exponent bits with bias 127, 7 fraction bits --
 *     the upper half of a binary32; field 0 holds zero and the subnormals
 *     f 2^-133, field 255 infinities and NaNs.
 *
 * Reading (listed with the design notes): the product of the decoded
 * inputs, C[i][j] = sum_k a_ik b_kj, summed like the fp32 oracle, k
 * ascending from +0.0 in binary64.  Each product of two 16-bit values has at
 * most 22 significant bits and is exact in binary64.  S = sum_k |a_ik b_kj|
 * is the scale of the acceptance bound.  Rounding fp32 data to 16 bits is
 * the caller's business and happens before the call.
 *
 * Pins (CPU tests): the decoders against numpy's binary16 and binary32
 * decoding for all 65,536 patterns; the product equal bit for bit to the
 * fp32 oracle on the same values widened to binary32; exact integer brute
 * force; closed forms; the formats' extreme values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

#define FMT_BF16 0
#define FMT_F16 1

/* The value of one 16-bit pattern, from its sign, exponent and fraction
 * fields. */
double oracle_decode16(int format, uint16_t bits)
{
    const int neg = bits >> 15;
    double v;
    if (format == FMT_BF16) {
        const int e = (bits >> 7) & 0xFF, f = bits & 0x7F;
        if (e == 0xFF)
            v = f ? NAN : INFINITY;
        else if (e == 0)
            v = ldexp((double)f, -133);             /* 2^(1-127) * f/2^7 */
        else
            v = ldexp(1.0 + f / 128.0, e - 127);
    } else {
        const int e = (bits >> 10) & 0x1F, f = bits & 0x3FF;
        if (e == 0x1F)
            v = f ? NAN : INFINITY;
        else if (e == 0)
            v = ldexp((double)f, -24);              /* 2^(1-15) * f/2^10 */
        else
            v = ldexp(1.0 + f / 1024.0, e - 15);
    }
    return neg ? -v : v;
}

int oracle_decode16_array(int format, int64_t n, const uint16_t *in, double *out)
{
    if ((format != FMT_BF16 && format != FMT_F16) || n < 0 || (n > 0 && (!in || !out)))
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < n; ++t)
        out[t] = oracle_decode16(format, in[t]);
    return ORACLE_OK;
}

/* Every pattern's value, so the dot products below look values up. */
static double *decode_table(int format)
{
    double *t = (double *)malloc(65536 * sizeof *t);
    if (t)
        for (int b = 0; b < 65536; ++b)
            t[b] = oracle_decode16(format, (uint16_t)b);
    return t;
}

/* c = sum_{k<K} a(i,k) b(k,j), s = sum_k |a(i,k) b(k,j)|, with a(i,k) =
 * value of A[i*a_rs + k*a_cs] and b(k,j) = value of B[k*b_rs + j*b_cs]: a
 * factor used as stored has strides (ld, 1), its transpose (1, ld). */
static void dot16(const double *val, int64_t K, const uint16_t *A, int64_t a_rs, int64_t a_cs,
                  const uint16_t *B, int64_t b_rs, int64_t b_cs, int64_t i, int64_t j,
                  double *c, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double prod = val[A[i * a_rs + k * a_cs]] * val[B[k * b_rs + j * b_cs]];
        acc += prod;
        mag += fabs(prod);
    }
    *c = acc;
    *s = mag;
}

struct rows16_job {
    const double *val;
    int64_t row_begin, row_end, N, K;
    const uint16_t *A; int64_t a_rs, a_cs;
    const uint16_t *B; int64_t b_rs, b_cs;
    double *C; int64_t ldc;
    double *S; int64_t lds;
};

static void *rows16_worker(void *arg)
{
    const struct rows16_job *job = (const struct rows16_job *)arg;
    for (int64_t i = job->row_begin; i < job->row_end; ++i)
        for (int64_t j = 0; j < job->N; ++j) {
            double c, s;
            dot16(job->val, job->K, job->A, job->a_rs, job->a_cs, job->B, job->b_rs, job->b_cs, i, j, &c, &s);
            job->C[i * job->ldc + j] = c;
            if (job->S)
                job->S[i * job->lds + j] = s;
        }
    return NULL;
}

/* Strides of op(X) for a stored row-major X with leading dimension ld: op 0
 * uses X as stored, op 1 its transpose. */
static void op16_strides(int op, int64_t ld, int64_t *rs, int64_t *cs)
{
    if (op == 0) { *rs = ld; *cs = 1; }
    else         { *rs = 1;  *cs = ld; }
}

/* C (binary64, leading dimension ldc) = op(A) x op(B) for 16-bit factors of
 * the given format.  op_a = 0: A stored M x K (lda >= K); op_a = 1: A stored
 * K x M (lda >= M).  op_b = 0: B stored K x N (ldb >= N); op_b = 1: B stored
 * N x K (ldb >= K).  S (optional) = sum of |products|.  Rows [row_begin,
 * row_end) only; threads split the rows, each element computed by one thread
 * with the same code. */
int oracle_gemm16_op_rows(int op_a, int op_b, int format, int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          double *C, int64_t ldc, double *S, int64_t lds,
                          int64_t row_begin, int64_t row_end, int threads)
{
    if (format != FMT_BF16 && format != FMT_F16)
        return ORACLE_BAD_ARG;
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || row_begin < 0 || row_end > M || row_begin > row_end)
        return ORACLE_BAD_ARG;
    const int64_t a_cols = op_a == 0 ? K : M, b_cols = op_b == 0 ? N : K;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if (S && lds < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if ((row_end > row_begin && N > 0) && (!C || (K > 0 && (!A || !B))))
        return ORACLE_BAD_ARG;
    int64_t a_rs, a_cs, b_rs, b_cs;
    op16_strides(op_a, lda, &a_rs, &a_cs);
    op16_strides(op_b, ldb, &b_rs, &b_cs);
    double *val = decode_table(format);
    int64_t rows = row_end - row_begin;
    if (threads < 1)
        threads = 1;
    if (threads > rows)
        threads = rows > 0 ? (int)rows : 1;
    struct rows16_job *jobs = (struct rows16_job *)calloc((size_t)threads, sizeof *jobs);
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof *tids);
    if (!val || !jobs || !tids) {
        free(val);
        free(jobs);
        free(tids);
        return ORACLE_BAD_ARG;
    }
    int64_t per = rows / threads, extra = rows % threads, r = row_begin;
    for (int t = 0; t < threads; ++t) {
        int64_t take = per + (t < extra ? 1 : 0);
        jobs[t] = (struct rows16_job){val, r, r + take, N, K, A, a_rs, a_cs, B, b_rs, b_cs, C, ldc, S, lds};
        r += take;
    }
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tids[t], NULL, rows16_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    rows16_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    for (int t = started + 1; t < threads; ++t)
        rows16_worker(&jobs[t]);
    free(val);
    free(jobs);
    free(tids);
    return ORACLE_OK;
}

/* The plain product A x B (both as stored), rows [row_begin, row_end). */
int oracle_gemm16_rows(int format, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       double *C, int64_t ldc, double *S, int64_t lds,
                       int64_t row_begin, int64_t row_end, int threads)
{
    return oracle_gemm16_op_rows(0, 0, format, M, N, K, A, lda, B, ldb, C, ldc, S, lds,
                                 row_begin, row_end, threads);
}

/* Selected entries (ii[t], jj[t]) of op(A) x op(B) only (op flags as in
 * oracle_gemm16_op_rows), for shapes too large for the full product. */
int oracle_gemm16_op_entries(int op_a, int op_b, int format, int64_t M, int64_t N, int64_t K,
                             const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                             int64_t count, const int64_t *ii, const int64_t *jj,
                             double *out_c, double *out_s)
{
    if (format != FMT_BF16 && format != FMT_F16)
        return ORACLE_BAD_ARG;
    if ((op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_BAD_ARG;
    const int64_t a_cols = op_a == 0 ? K : M, b_cols = op_b == 0 ? N : K;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1))
        return ORACLE_BAD_ARG;
    if (count > 0 && (!ii || !jj || !out_c || !out_s || (K > 0 && (!A || !B))))
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < count; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return ORACLE_BAD_ARG;
    int64_t a_rs, a_cs, b_rs, b_cs;
    op16_strides(op_a, lda, &a_rs, &a_cs);
    op16_strides(op_b, ldb, &b_rs, &b_cs);
    double *val = decode_table(format);
    if (!val)
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < count; ++t)
        dot16(val, K, A, a_rs, a_cs, B, b_rs, b_cs, ii[t], jj[t], &out_c[t], &out_s[t]);
    free(val);
    return ORACLE_OK;
}

int oracle_gemm16_entries(int format, int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          int64_t count, const int64_t *ii, const int64_t *jj,
                          double *out_c, double *out_s)
{
    return oracle_gemm16_op_entries(0, 0, format, M, N, K, A, lda, B, ldb, count, ii, jj, out_c, out_s);
}
