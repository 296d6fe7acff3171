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
 * value of A[i*lda + k] and b(k,j) = value of B[k*ldb + j]. */
static void dot16(const double *val, int64_t K, const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb, int64_t i, int64_t j, double *c, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double prod = val[A[i * lda + k]] * val[B[k * ldb + j]];
        acc += prod;
        mag += fabs(prod);
    }
    *c = acc;
    *s = mag;
}

struct rows16_job {
    const double *val;
    int64_t row_begin, row_end, N, K;
    const uint16_t *A; int64_t lda;
    const uint16_t *B; int64_t ldb;
    double *C; int64_t ldc;
    double *S; int64_t lds;
};

static void *rows16_worker(void *arg)
{
    const struct rows16_job *job = (const struct rows16_job *)arg;
    for (int64_t i = job->row_begin; i < job->row_end; ++i)
        for (int64_t j = 0; j < job->N; ++j) {
            double c, s;
            dot16(job->val, job->K, job->A, job->lda, job->B, job->ldb, i, j, &c, &s);
            job->C[i * job->ldc + j] = c;
            if (job->S)
                job->S[i * job->lds + j] = s;
        }
    return NULL;
}

/* C (binary64, leading dimension ldc) = A x B for 16-bit A (M x K, lda >= K)
 * and B (K x N, ldb >= N) of the given format; S (optional) = sum of
 * |products|.  Rows [row_begin, row_end) only; threads split the rows, each
 * element computed by one thread with the same code. */
int oracle_gemm16_rows(int format, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       double *C, int64_t ldc, double *S, int64_t lds,
                       int64_t row_begin, int64_t row_end, int threads)
{
    if (format != FMT_BF16 && format != FMT_F16)
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || row_begin < 0 || row_end > M || row_begin > row_end)
        return ORACLE_BAD_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if (S && lds < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if ((row_end > row_begin && N > 0) && (!C || (K > 0 && (!A || !B))))
        return ORACLE_BAD_ARG;
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
        jobs[t] = (struct rows16_job){val, r, r + take, N, K, A, lda, B, ldb, C, ldc, S, lds};
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

/* Selected entries (ii[t], jj[t]) of A x B only, for shapes too large for
 * the full product on the host. */
int oracle_gemm16_entries(int format, int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          int64_t count, const int64_t *ii, const int64_t *jj,
                          double *out_c, double *out_s)
{
    if (format != FMT_BF16 && format != FMT_F16)
        return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_BAD_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if (count > 0 && (!ii || !jj || !out_c || !out_s || (K > 0 && (!A || !B))))
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < count; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return ORACLE_BAD_ARG;
    double *val = decode_table(format);
    if (!val)
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < count; ++t)
        dot16(val, K, A, lda, B, ldb, ii[t], jj[t], &out_c[t], &out_s[t]);
    free(val);
    return ORACLE_OK;
}
