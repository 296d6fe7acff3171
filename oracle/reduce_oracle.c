/*
 * reduce_oracle.c -- the CPU oracle for the sum reduction and for the
 * bookkeeping of the tree reductions.
 *
 * TEST INFRASTRUCTURE ONLY, like gemm_oracle.c: nothing in the product path
 * may include, link, load or call it.
 *
 * What it follows: "03 CUDA Shared Memory: Tiling, Bank Conflicts, and
 * Reduction", section "Reduction":
 *   - a reduction folds N values into one; for a sum, the result is
 *     x_0 + x_1 + ... + x_{N-1};
 *   - a tree of pairwise additions takes log2 N steps and still N - 1
 *     additions;
 *   - version 0 lets thread tid add at step s when tid % (2s) == 0, version 1
 *     when tid < s (sequential addressing); the page counts, per step, the
 *     warps that hold at least one adding thread (47 in total for version 0
 *     against 12 for version 1, for 256 elements and 32-thread warps);
 *   - the multi-pass scheme reduces blocks of values to one partial each and
 *     runs again on the partials until one value is left (2^24 values with
 *     256 per block: 65,536, then 256, then 1 -- three launches).
 *
 * Readings: the sum is taken in binary64, indices ascending from +0.0 (the
 * plain definition; every binary32 input is exact in binary64); alongside it
 * the oracle returns sum |x_i|, the scale of the GPU's error bound.
 *
 * Pins (CPU tests): exact integer sums, closed forms, the exact float sum
 * (math.fsum) within n 2^-53 sum |x|, and the page's printed step, addition,
 * warp and launch counts.
 */
#include <math.h>
#include <stdint.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* *sum = x_0 + ... + x_{n-1} and *abs_sum = |x_0| + ... in binary64, in
 * index order from +0.0. */
int oracle_sum(int64_t n, const float *x, double *sum, double *abs_sum)
{
    if (n < 0 || (n > 0 && !x) || !sum)
        return ORACLE_BAD_ARG;
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s += (double)x[i];
        a += fabs((double)x[i]);
    }
    *sum = s;
    if (abs_sum)
        *abs_sum = a;
    return ORACLE_OK;
}

/* Bookkeeping of one block's tree reduction over `block` values (a power of
 * two) by `block` threads in warps of `warp` threads.
 *   version 0: at step s = 1, 2, 4, ..., thread tid adds when tid % (2s) == 0
 *   version 1: at step s = block/2, ..., 2, 1, thread tid adds when tid < s
 * out[0] = steps, out[1] = additions, out[2] = sum over steps of the number of
 * warps holding at least one adding thread. */
int oracle_tree_counts(int64_t block, int64_t warp, int version, int64_t *out)
{
    if (block < 1 || (block & (block - 1)) != 0 || warp < 1 || (version != 0 && version != 1) || !out)
        return ORACLE_BAD_ARG;
    int64_t steps = 0, adds = 0, warp_steps = 0;
    for (int64_t k = 1; k < block; k *= 2) {
        const int64_t s = version == 0 ? k : block / (2 * k);
        int64_t warps_here = 0;
        for (int64_t w = 0; w * warp < block; ++w) {
            int any = 0;
            for (int64_t tid = w * warp; tid < (w + 1) * warp && tid < block; ++tid) {
                const int active = version == 0 ? (tid % (2 * s) == 0) : (tid < s);
                if (active) {
                    adds++;
                    any = 1;
                }
            }
            warps_here += any;
        }
        warp_steps += warps_here;
        steps++;
    }
    out[0] = steps;
    out[1] = adds;
    out[2] = warp_steps;
    return ORACLE_OK;
}

/* The multi-pass scheme: each launch turns n values into ceil(n / per_block)
 * partials, until one value is left.  sizes[0] = n, sizes[i] = the count
 * after launch i (up to max_sizes entries); returns the number of launches,
 * or -1 on bad arguments. */
int64_t oracle_reduce_passes(int64_t n, int64_t per_block, int64_t *sizes, int64_t max_sizes)
{
    if (n < 1 || per_block < 2 || (max_sizes > 0 && !sizes))
        return -1;
    int64_t launches = 0;
    if (max_sizes > 0)
        sizes[0] = n;
    while (n > 1) {
        n = (n + per_block - 1) / per_block;
        launches++;
        if (launches < max_sizes)
            sizes[launches] = n;
    }
    return launches;
}
