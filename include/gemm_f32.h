/*
 * gemm_f32.h -- C ABI of the MI355X (gfx950) fp32 matrix-product library.
 *
 * The operation is the dense product C = A x B of the pages on shared-memory
 * tiling ("03 CUDA Shared Memory: Tiling, Bank Conflicts, and Reduction",
 * section "Shared Memory와 Tiling"; PMPP chapter 5 notes
 * "메모리 계층과 데이터 지역성", sections 5.4 and 5.5): every output element is
 * the dot product of one row of A with one column of B, matrices are stored
 * row by row, sizes need not be multiples of the tile because out-of-range
 * tile slots hold zero, and only the final store is range checked.  The pages
 * state it for square Width x Width matrices; this interface takes the
 * general M x K times K x N case with BLAS-style leading dimensions (an
 * offset sub-matrix view is a base pointer plus a leading dimension, as in
 * the first page's "Global Memory와 Coalescing" section).
 *
 * Layout (all three matrices row-major, binary32):
 *   A is M x K,  element (i, k) at A[i*lda + k],  lda >= max(1, K)
 *   B is K x N,  element (k, j) at B[k*ldb + j],  ldb >= max(1, N)
 *   C is M x N,  element (i, j) at C[i*ldc + j],  ldc >= max(1, N)
 *
 * Result: C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j] for i < M,
 * j < N, rounded in binary32 (summation order and fused multiply-adds vary
 * by kernel; see the accuracy note below).  C is OVERWRITTEN (no alpha, no
 * beta, C is never read).  Entries of C outside the M x N window -- the
 * padding between N and ldc -- are never written.  K == 0 writes +0 to the
 * whole window.  M == 0 or N == 0 is a no-op that returns GEMM_F32_OK.
 *
 * Memory and ownership: A, B and C are DEVICE pointers on the current HIP
 * device, owned by the caller; the library allocates nothing, keeps no
 * pointer after returning and holds no state (the one exception is the
 * fixed 1 MiB scratch array of reduce_sum_f32_variant_noalloc, a static
 * device variable, and its address per device).  A and B are read only.  C
 * must not overlap A or B (the result is undefined otherwise).  Pointers need
 * 4-byte alignment only; 16-byte alignment is not required.
 *
 * Streams and errors: `stream` is a hipStream_t (NULL = the null stream).
 * Every call only enqueues work: it returns before the product is computed,
 * and the caller synchronises the stream to see the result.  Argument errors
 * are detected synchronously, before anything is enqueued, and are returned
 * as a nonzero status with no launch.  GEMM_F32_ERR_LAUNCH reports a launch
 * rejected by the HIP runtime; a fault during execution surfaces at the
 * caller's next synchronisation, as for any HIP kernel.  All entry points are
 * thread safe.
 *
 * Accuracy: the result of every kernel satisfies, per element,
 *   |C - C_exact| <= 1e-5 * sum_k |A_ik| |B_kj|
 * on the workloads the library is tested on, and is bit exact whenever every
 * product and partial sum is an integer below 2^24 in magnitude (for
 * instance small-integer inputs).
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every entry point returns one, synchronously, before it
 * enqueues anything: the host-program habit of the one-volume PMPP notes
 * ("PMPP 단권화", chapter 2, host program structure), which checks the
 * status of every runtime call and reports it by name, carried over to the
 * library's own argument checks.  The codes and their texts
 * (gemm_f32_status_string) are this library's own. */
#define GEMM_F32_OK                  0
#define GEMM_F32_ERR_INVALID_DIM     1  /* M, N or K negative                       */
#define GEMM_F32_ERR_INVALID_LD      2  /* lda < max(1,K), ldb or ldc < max(1,N)     */
#define GEMM_F32_ERR_NULL_PTR        3  /* a pointer is NULL while its matrix is non-empty */
#define GEMM_F32_ERR_MISALIGNED      4  /* a pointer is not 4-byte aligned           */
#define GEMM_F32_ERR_INVALID_VARIANT 5  /* unknown kernel variant                    */
#define GEMM_F32_ERR_TOO_LARGE       6  /* M, N or K >= 2^31, or the grid would not fit */
#define GEMM_F32_ERR_LAUNCH          7  /* the HIP runtime rejected the launch       */
#define GEMM_F32_ERR_DEVICE          8  /* no usable current HIP device              */
#define GEMM_F32_ERR_INVALID_OP      9  /* op_a or op_b is neither N nor T           */
#define GEMM_F32_ERR_WORKSPACE      10  /* workspace smaller than required            */
#define GEMM_F32_ERR_INVALID_FORMAT 11  /* 16-bit input format unknown                */
#define GEMM_F32_ERR_SCRATCH        12  /* partials would exceed the fixed scratch      */

/* Kernel ladder.  Each rung computes the same product; each is tested against
 * the oracle and against the rung below it.
 *   0  naive: one thread per output element, 16 x 16 workgroups, operands read
 *      straight from global memory (PMPP one-volume notes, naive matrix
 *      product; first page, naive kernel)
 *   1  LDS-tiled: the pages' tiled kernel with T = 32 -- 32 x 32 A and B tiles
 *      staged cooperatively in LDS with ghost zeros, two barriers per phase,
 *      rows padded by 4 words, 128-bit coalesced global loads
 *   2  register-blocked, double-buffered: 128 x 128 workgroup tile, 8 x 8
 *      outputs per thread in registers, two LDS buffers and one barrier per
 *      phase, next tile prefetched into registers during the current phase
 *   3  MFMA: v_mfma_f32_32x32x2_f32 matrix-core contraction on double-
 *      buffered LDS tiles (the default).  The tile follows from how full the
 *      last round of 256 workgroups would run: 256 x 256 tiles with direct
 *      global-to-LDS copies into an XOR-swizzled layout (on four waves with
 *      a fixed instruction order when K, M and N are multiples of 4
 *      and each stored factor is under 2 GiB, else on eight waves; both give
 *      the same bits), else 128 x 128 tiles, else 64 x 64 tiles whose phases
 *      are split over four groups of four waves.  With K, M and N multiples
 *      of 4, 64 x 64 tiles whose four waves each run the whole tile over
 *      every fourth phase (partial tiles added in wave order, so results are
 *      deterministic and the same for every op pair) replace that choice
 *      where a cost model of rounds, per-kernel efficiency and fixed cost
 *      per tile gives them the shorter time (K >= 448), or in place of the
 *      split-phase tiles (K >= 384); then 96 x 96 tiles of the same kind
 *      (16-deep phases) where the model gives them the shorter time (K >=
 *      448), and, from K = 256, 64 x 64 tiles of four waves with one 32 x
 *      32 block each over the whole K (three blocks sharing a CU) where the
 *      model, charging their fixed cost once per launch, does.  Products of at most 1024 output tiles
 *      of 16 x 16 take small tiles instead (16 x 16 on 8 waves up to 512 of
 *      them, else 32 x 32 on 4 waves), whose K is split over the waves of
 *      each block, operands loaded straight into registers for
 *      v_mfma_f32_16x16x4_f32, partial tiles added in wave order.
 *      gemm_f32_default_variant() names the configuration a shape runs.
 * Variants numbered from 16 up are diagnostic layouts of the same rungs, kept
 * so that their hardware counters can be compared; see
 * gemm_f32_variant_name().
 */
#define GEMM_F32_VARIANT_NAIVE    0
#define GEMM_F32_VARIANT_TILED    1
#define GEMM_F32_VARIANT_REGBLOCK 2
#define GEMM_F32_VARIANT_MFMA     3

/* C = A x B with the library's best kernel for the shape (the MFMA rung). */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/* Same contract, with the kernel chosen by `variant` (see above).
 * Returns GEMM_F32_ERR_INVALID_VARIANT for an unknown number. */
int gemm_f32_variant(int variant,
                     int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     void *stream);

/* Products with a transposed factor: C = op(A) x op(B), C still M x N.
 *
 * The one-volume PMPP notes (deep-learning chapter, backward pass) need the
 * weight gradient X^T dY and the input gradient dY W^T besides the forward
 * product, and run all three on the same tile kernel; so does this entry
 * point (the MFMA rung, with each factor's LDS tile kept in the orientation
 * in which it is stored).
 *   op_a == GEMM_F32_OP_N: A is stored M x K, element (i,k) at A[i*lda + k],
 *                          lda >= max(1, K)
 *   op_a == GEMM_F32_OP_T: A is stored K x M, element (i,k) of op(A) at
 *                          A[k*lda + i], lda >= max(1, M)
 *   op_b == GEMM_F32_OP_N: B is stored K x N, element (k,j) at B[k*ldb + j],
 *                          ldb >= max(1, N)
 *   op_b == GEMM_F32_OP_T: B is stored N x K, element (k,j) of op(B) at
 *                          B[j*ldb + k], ldb >= max(1, K)
 * C, ownership, streams, errors and accuracy are as for gemm_f32; an op
 * other than N or T returns GEMM_F32_ERR_INVALID_OP.  For a given M, N, K
 * the k-summation order does not depend on the ops, so op(A) = A^T gives
 * the same bits as gemm_f32 on an explicitly transposed copy.
 */
#define GEMM_F32_OP_N 0
#define GEMM_F32_OP_T 1
int gemm_f32_op(int op_a, int op_b,
                int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream);

/* Introspection.  These calls are this library's own (the pages define no
 * such interface): they launch nothing, need no device, and exist so that
 * tests, benchmarks and counter runs can name the kernels they measure.
 *
 * Number of ladder rungs (variants 0 .. n-1). */
int gemm_f32_num_variants(void);

/* Static, NUL-terminated name of a variant, or NULL if it does not exist.
 * Valid numbers are 0 .. gemm_f32_num_variants()-1 and the diagnostic
 * numbers 16 .. 16 + gemm_f32_num_diagnostic_variants() - 1. */
const char *gemm_f32_variant_name(int variant);

/* Number of diagnostic variants (numbered from 16). */
int gemm_f32_num_diagnostic_variants(void);

/* The diagnostic variant whose configuration gemm_f32 and gemm_f32_op run
 * for an M x N x K product (the choice depends on the sizes only; the
 * four-wave configuration hands a stored factor of 2 GiB or more to the
 * eight-wave kernel), or -1 for sizes that are
 * negative or above INT_MAX.  Launches nothing, needs no device; for callers
 * that want to know which kernel a call will use. */
int gemm_f32_default_variant(int64_t M, int64_t N, int64_t K);

/* Measurement helper, this library's own (not part of the product): a loop
 * of non-packed binary32 fused multiply-adds on the vector ALU -- the
 * register-blocked rung's instruction -- whose time, measured by the caller,
 * gives that instruction's issue rate on the device.
 *   form    0: one operand in a scalar register; 1: all operands in vector
 *           registers, 16 independent accumulators per lane; 2: an 8 x 8
 *           outer product of vector registers (the rung's inner step)
 *   blocks  workgroups of 256 threads (4 waves) to launch, >= 1
 *   iters   loop trips: each lane does iters x 16 FMAs (forms 0 and 1) or
 *           (iters / 4) x 64 (form 2)
 *   out     device pointer to blocks x 256 floats, overwritten (keeps the
 *           results live)
 *   stamps  device pointer to blocks x 4 x 4 uint64_t (8-byte aligned): for
 *           wave w, stamps[4w .. 4w+3] = shader clock counter and 100 MHz
 *           counter at the start, then at the end of its loop
 * Enqueue-only on `stream`; statuses as for gemm_f32 (an unknown form gives
 * GEMM_F32_ERR_INVALID_VARIANT). */
int gemm_f32_valu_probe(int form, int64_t blocks, int iters, float *out, uint64_t *stamps,
                        void *stream);

/* Measurement helper, this library's own (not part of the product): one
 * wave (a single workgroup of 64 threads) reads LDS, lane l at byte offset
 * offsets[l] of a 64 KB array (masked into it and aligned down to the read's
 * width), `iters` times; with a profiler's LDS bank-conflict counter per
 * dispatch, a chosen set of offsets shows which lanes one read cycle serves.
 *   form     0 ds_read_b32, 1 ds_read_b64, 2 ds_read_b128,
 *            3 ds_read_b64_tr_b16
 *   offsets  device pointer to 64 int32 byte offsets (4-byte aligned)
 *   out      device pointer to 64 uint32, overwritten (keeps the reads live)
 * Enqueue-only on `stream`; statuses as for gemm_f32 (an unknown form gives
 * GEMM_F32_ERR_INVALID_VARIANT, iters < 0 GEMM_F32_ERR_INVALID_DIM). */
int gemm_f32_lds_probe(int form, const int32_t *offsets, int iters, uint32_t *out, void *stream);

/* Measurement helper, this library's own (not part of the product): the
 * rate at which a CU brings 1 KB wave loads (16 bytes a lane, as the 16-bit
 * kernels' copies) from an L2-resident buffer, into LDS or into registers.
 * Each workgroup (4 waves) reads its own 64 KB of src, wave w the 16 KB at
 * 16 KB w, cycling through it `iters` x 8 times with 8 to 16 loads in flight.
 *   mode    0: buffer loads into LDS; 1: buffer loads into vector registers
 *   blocks  workgroups of 256 threads, >= 1 (one per CU for a per-CU rate)
 *   iters   loop trips, even, >= 0
 *   src     device pointer, 16-byte aligned, to blocks x 65536 bytes
 *           (blocks x 64 KB should fit the L2 caches)
 *   out     device pointer to blocks x 256 uint32, overwritten
 *   cycles  device pointer to blocks x 4 uint64 (8-byte aligned): each
 *           wave's shader clock cycles for its loop
 * Enqueue-only on `stream`; statuses as for gemm_f32 (an unknown mode gives
 * GEMM_F32_ERR_INVALID_VARIANT, odd or negative iters
 * GEMM_F32_ERR_INVALID_DIM). */
int gemm_f32_copy_probe(int mode, int64_t blocks, int iters, const void *src, uint32_t *out, uint64_t *cycles,
                        void *stream);

/* Measurement helper, this library's own (no page defines it): gemm_f32's
 * k-split kernel (64 x 64 tiles whose four waves each take every fourth
 * phase of the tile; gemm_f32 runs it for square1000-sized products) on an
 * instantiation that also records when each wave passes five points.  A, B,
 * C and every size, leading dimension and status as for gemm_f32 with both
 * factors as stored; C receives the same bits as gemm_f32 gives with the
 * k-split kernel.  The problem must be one that kernel takes (M, N, K
 * multiples of 4, K > 0, M and N > 0), else GEMM_F32_ERR_INVALID_DIM.
 *   timeline        device buffer of timeline_words uint32 words, 4-byte
 *                   aligned; timeline_words a positive multiple of 32
 *                   (GEMM_F32_ERR_INVALID_DIM otherwise)
 * Block b < timeline_words / 32 (in launch order), wave w, writes words
 * 8 (4 b + w) .. + 7: the 100 MHz real-time counter at the wave's start,
 * when its first phase has landed in LDS, after its last matrix instruction
 * is issued, after the barrier before the partial tiles are added, and after
 * its stores have completed; its shader-clock cycles between the first and
 * the last; its phase count; b.  Other words are not written.  The
 * instantiation waits for its stores before the last stamp, which the
 * product kernel does not.  Enqueue-only on `stream`. */
int gemm_f32_ksplit_timeline(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                             int64_t ldb, float *C, int64_t ldc, uint32_t *timeline, int64_t timeline_words,
                             void *stream);

/* Static, NUL-terminated description of a status code (the by-name report
 * of the chapter 2 error check cited with the codes above); "unknown status"
 * for any other number. */
const char *gemm_f32_status_string(int status);

/* Shared-tile transpose: out = in^T, binary32, row-major.
 *
 * The first page's "Bank Conflict" section transposes through a tile held
 * in shared memory -- read rows of `in` and write rows of `out`, both
 * coalesced, reading the tile by columns in between -- and uses it to show
 * bank conflicts and their cures (padding, XOR swizzle).
 *   in  is rows x cols, element (r, c) at in[r*ld_in + c],   ld_in  >= max(1, cols)
 *   out is cols x rows, element (c, r) at out[c*ld_out + r], ld_out >= max(1, rows)
 * out[c*ld_out + r] = in[r*ld_in + c] exactly; words of out outside the
 * cols x rows window are never written.  Device pointers, caller-owned, 4-byte
 * aligned; out must not overlap in.  rows or cols == 0 is a no-op.  Status
 * codes, streams and asynchrony as for gemm_f32 (GEMM_F32_ERR_INVALID_LD for
 * a too-small leading dimension, GEMM_F32_ERR_INVALID_VARIANT for an unknown
 * variant).
 * Variants: 0 naive (no LDS), 1 [32][32] tile (the page's kernel), 2 [32][33]
 * padded tile, 3 XOR-swizzled [32][32] tile, 4 64 x 64 tile with 128-bit
 * global and LDS accesses and an LDS layout conflict free on gfx950, 5 the
 * same with 128 x 128 tiles, 6 variant 4 with tiles handed out in diagonal
 * order, 7 and 8 variants 6 and 4 with nontemporal global loads and stores,
 * 9 and 10 variant 6 and its 128 x 128 form with nontemporal stores only.
 * transpose_f32 uses 9 when the 64 x 64 tile grid is square or the input
 * holds 128 MiB or more, else 6 (diagonal order: with leading dimensions
 * near a multiple of 4 KB, tiles handed out row by row crowd the same memory
 * channels; nontemporal stores keep the caches for the input);
 * transpose_f32_default_variant names that choice (-1 for negative sizes or
 * sizes above INT_MAX), launching nothing.
 */
int transpose_f32(int64_t rows, int64_t cols, const float *in, int64_t ld_in,
                  float *out, int64_t ld_out, void *stream);
int transpose_f32_variant(int variant, int64_t rows, int64_t cols, const float *in,
                          int64_t ld_in, float *out, int64_t ld_out, void *stream);
int transpose_f32_num_variants(void);
const char *transpose_f32_variant_name(int variant);   /* NULL if unknown */
int transpose_f32_default_variant(int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out);

/* Sum reduction: *out = x[0] + ... + x[n-1], binary32.
 *
 * The first page's "Reduction" section folds an array into one value with a
 * tree in shared memory, improves the tree step by step (interleaved, then
 * sequential addressing, then warp shuffles for the last steps, then one
 * atomic per block), and reduces large arrays in several passes (each block
 * folds its values to one partial, then the partials are folded again).
 *   x          device pointer to n floats (4-byte aligned), read only
 *   out        device pointer to one float, overwritten (+0 when n == 0)
 *   workspace  device memory of at least reduce_sum_f32_workspace_size()
 *              bytes for the partials (NULL allowed when that size is 0);
 *              owned by the caller, contents undefined after the call; it
 *              must not overlap x or out
 * The summation order depends on the variant and on n only, except for
 * variant 3, whose block sums are added by float atomics in arrival order:
 * its last bits may vary from run to run.  The error is bounded by
 * (longest sequential chain + tree depth) * 2^-24 * sum |x_i|; the result is
 * exact when every partial sum is an integer below 2^24 in magnitude.
 * Variants: 0 interleaved pairs (the thread owning a pair's left slot adds),
 * 1 sequential addressing (the lowest-numbered threads add), 2 sequential +
 * wave shuffles for the last six steps, 3 one atomic add per block, 4
 * grid-stride 128-bit loads + wave shuffles + a one-block second pass (the
 * default).  Statuses as for gemm_f32, plus GEMM_F32_ERR_WORKSPACE.
 */
int64_t reduce_sum_f32_workspace_size(int variant, int64_t n);   /* bytes; -1 if invalid */
int reduce_sum_f32(int64_t n, const float *x, float *out,
                   void *workspace, int64_t workspace_bytes, void *stream);
int reduce_sum_f32_variant(int variant, int64_t n, const float *x, float *out,
                           void *workspace, int64_t workspace_bytes, void *stream);
int reduce_sum_f32_num_variants(void);
const char *reduce_sum_f32_variant_name(int variant);  /* NULL if unknown */

/* reduce_sum_f32_variant without a workspace, for callers that cannot
 * allocate device memory: code under HIP stream capture, serving loops that
 * must not call the allocator, harnesses that forbid it.  It calls no
 * allocator (the library's, HIP's or torch's) at any point.
 *   The partials go to a fixed array of REDUCE_SUM_F32_SCRATCH_BYTES (1 MiB)
 * that the library holds in the device memory of every GPU it runs on, for
 * the life of the process.  Its address on a device is looked up on the
 * first call with that device current.
 *   Limit: a problem whose partials need more than that scratch, i.e. whose
 * reduce_sum_f32_workspace_size(variant, n) exceeds
 * REDUCE_SUM_F32_SCRATCH_BYTES, is rejected with GEMM_F32_ERR_SCRATCH
 * before anything is enqueued.  Variants 3 and 4 fit for any n; variants
 * 0-2 need about 4 n / 255 bytes, so they take n up to about 6.7e7.
 *   Sharing: every call on one GPU uses that GPU's one scratch array, which
 * keeps the last call's contents.  Calls that overlap on one GPU -- on two
 * streams, or from two host threads without ordering -- race and give
 * undefined results.  Calls on one stream are ordered and safe.
 *   Arguments, results, summation order (the same bits as
 * reduce_sum_f32_variant for variants 0-2 and 4), statuses and asynchrony
 * are as for reduce_sum_f32_variant. */
#define REDUCE_SUM_F32_SCRATCH_BYTES (1 << 20)
int reduce_sum_f32_variant_noalloc(int variant, int64_t n, const float *x, float *out,
                                   void *stream);

/* Mixed-precision product: C (binary32) = A x B with A and B in a 16-bit
 * format, accumulated in binary32.
 *
 * The one-volume PMPP notes ("PMPP 단권화", deep-learning chapter, "FC Layer
 * = GEMM" and "Mixed Precision") run the fully connected layer as a matrix
 * product on matrix units that take FP16 or BF16 inputs and accumulate in
 * FP32; BF16 keeps FP32's exponent range, FP16 does not.
 *   format   GEMM_MIXED_BF16 (bfloat16: 1 sign, 8 exponent, 7 fraction bits)
 *            or GEMM_MIXED_F16 (IEEE binary16: 1 sign, 5 exponent, 10
 *            fraction bits); both factors use the same format
 *   A        M x K, element (i, k) at A[i*lda + k], lda >= max(1, K), 16-bit
 *            patterns, 2-byte aligned
 *   B        K x N, element (k, j) at B[k*ldb + j], ldb >= max(1, N), same
 *   C        M x N binary32, element (i, j) at C[i*ldc + j], ldc >= max(1, N),
 *            4-byte aligned
 * Leading dimensions count elements.  C[i*ldc + j] = sum_k a_ik b_kj: every
 * product of two 16-bit values is exact in binary32, the sum is accumulated
 * in binary32 (the accuracy bound of gemm_f32 applies, measured against the
 * exact product of the 16-bit values), and the result is bit exact whenever
 * every partial sum is an integer below 2^24 in magnitude.  Rounding binary32
 * data to 16 bits is the caller's step, before the call.  Overwrite, window,
 * K == 0, empty-size, ownership, stream and error rules as for gemm_f32; an
 * unknown format returns GEMM_F32_ERR_INVALID_FORMAT.  Operands whose bases
 * are 4-byte aligned with even leading dimensions use vector loads; others
 * are served by element-wise loads (correct, slower).
 * gemm_mixed picks the tile shape for the problem; gemm_mixed_variant runs
 * tile configuration `variant` (0 .. gemm_mixed_num_variants() - 1, named by
 * gemm_mixed_variant_name).  Below 128 tiles of 128 x 128 (and below 128 of
 * 256 x 256) with K a multiple of 8, gemm_mixed and gemm_mixed_op take
 * 64 x 64 tiles whose four waves each run the whole tile over every fourth
 * 32-deep phase (mixed64x64_bk32_w4_ksplit, v_mfma_f32_16x16x32; partial
 * tiles added in wave order, so every op pair gives the same bits); it needs
 * what the scheduled configurations need (below), and a problem it does not
 * take runs the element-wise 64 x 64 kernel.  With 128 to 256 tiles of
 * 128 x 128 and K >= 1024 (a multiple of 8) they take the same split on
 * 128 x 128 tiles (mixed128x128_bk32_w4_ksplit), with the same needs; a
 * problem it does not take runs mixed128x128_bk64_w2x2_directAB (aligned) or
 * the element-wise 128 x 128 kernel.  The scheduled configurations
 * -- mixed256x256_bk64_w4_wide (v_mfma_f32_16x16x32; gemm_mixed's and
 * gemm_mixed_op's choice once there are 128 tiles of 256 x 256),
 * mixed192x192_bk64_w4_wide (the same kernel on 192 x 192 tiles; their
 * choice, with K even, where its tiles need fewer rounds of the 256 CUs at
 * 0.8 of a 256 tile's time each, or, below 128 tiles of 256 x 256, with at
 * least 140 of 192 x 192 or, for K % 8 != 0, 32 of them with K < 1536 (or
 * K % 4 == 2 and fewer than 128 tiles of 128 x 128)),
 * mixed160x160_bk64_w4_wide (the same kernel on 160 x 160 tiles; their
 * choice wherever 192 x 192 tiles would be, if the 160 x 160 ones need no
 * more rounds of the 256 CUs),
 * mixed256x256_rowsplit (their choice, with K a multiple of 8, where the
 * last round of 256 x 256 tiles would be under 40 % full: the rows filling
 * the other rounds on the 256 x 256 kernel, the remaining rows on k-split
 * 128 x 128 tiles if at most 256 of them, else on 160 x 160 tiles if they
 * need no more rounds of the 256 CUs than 192 x 192 ones, else on 192 x 192
 * tiles; two launches in stream order),
 * mixed256x256_bk64_w4_sched (the same schedule on v_mfma_f32_32x32x16) and
 * mixed256x256_bk32_w4_wide4stage (16x16x32 with four 32-deep LDS stages) --
 * take K a multiple of 8 (the 16x16x32 wide ones on 256, 192 and 160 tiles: K even), N even (M
 * too for A stored transposed in gemm_mixed_op, and not N for B stored
 * transposed), 4-byte aligned operands with even leading dimensions and
 * operands under 2^31 bytes; edge tiles run whole and store only inside C,
 * and k positions past K contribute zeros.  Other
 * problems given to them run mixed256x256_bk64_w2x4_directAB (for the
 * 32 x 32 x 16 configuration the same tiles and summation order, the same
 * bits; for the 16 x 16 x 32 ones another instruction, other bits within the
 * same bound).
 */
#define GEMM_MIXED_BF16 0
#define GEMM_MIXED_F16  1

int gemm_mixed(int format, int64_t M, int64_t N, int64_t K,
               const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
               float *C, int64_t ldc, void *stream);
int gemm_mixed_variant(int variant, int format, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       float *C, int64_t ldc, void *stream);
int gemm_mixed_num_variants(void);
const char *gemm_mixed_variant_name(int variant);   /* NULL if unknown */
/* The configuration gemm_mixed runs for an M x N x K product (the scheduled
 * configurations hand problems they do not take to
 * the 8-wave fallback, as described above), or -1 for sizes that are negative
 * or above INT_MAX.  Launches nothing, needs no device. */
int gemm_mixed_default_variant(int64_t M, int64_t N, int64_t K);

/* C (binary32) = op(A) x op(B) for 16-bit factors, either one stored
 * transposed: the backward-pass products X^T dY and dY W^T of the same
 * deep-learning chapter ("Backward"), in mixed precision.
 *   op_a = GEMM_F32_OP_N: A stored M x K (lda >= max(1, K));
 *   op_a = GEMM_F32_OP_T: A stored K x M (lda >= max(1, M)), op(A) = A^T;
 *   op_b = GEMM_F32_OP_N: B stored K x N (ldb >= max(1, N));
 *   op_b = GEMM_F32_OP_T: B stored N x K (ldb >= max(1, K)), op(B) = B^T.
 * Everything else as for gemm_mixed (formats, alignment, accuracy, errors;
 * GEMM_F32_ERR_INVALID_OP for another op value).  The factors are read in
 * place; for a given M, N and K the result has the same bits whichever way
 * the factors are stored, as long as each storage meets the conditions of
 * the configuration gemm_mixed picks: from 128 tiles of 256 x 256 on, a
 * storage that does not (an odd M for A stored transposed, an odd N for B
 * as stored, an odd leading dimension, a 2-byte aligned base) runs the
 * 8-wave fallback on v_mfma_f32_32x32x16, whose bits differ within the same
 * bound. */
int gemm_mixed_op(int op_a, int op_b, int format, int64_t M, int64_t N, int64_t K,
                  const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                  float *C, int64_t ldc, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
