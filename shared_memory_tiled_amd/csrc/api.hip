// api.hip -- the C-ABI entry points declared in include/gemm_f32.h.
//
// Argument checking follows the error-checking habit of the PMPP one-volume
// notes (host program structure: every runtime call's status is checked):
// every error is reported as a status code, synchronously, before anything
// is enqueued.  The degenerate sizes follow the tiled kernel's phase loop
// (PMPP chapter 5 notes, section 5.4): with K = 0 there are no phases and
// every output is the initial +0; with M = 0 or N = 0 there is no output.
#include "gemm_f32.h"
#include "launch.h"

#include <limits.h>

namespace gemmf32 {
namespace {

constexpr int kNumRungs = 4;
constexpr int kDiagBase = 16;

// Diagnostic variants (numbered from 16): same rungs, other layouts or tile
// shapes, built so their hardware counters can be compared.
struct Diagnostic { const char* name; int rung; int config; };
const Diagnostic kDiagnostics[] = {
    {"tiled32_pad0", 1, 0},
    {"tiled32_pad1", 1, 1},
    {"regblock128x128_bk8_padA0", 2, 1},
    {"regblock128x128_bk16_padA4", 2, 2},
    {"mfma256x256_bk16_w2x2", 3, 0},
    {"mfma128x128_bk16_w2x2", 3, 1},
    {"mfma256x128_bk16_w2x2", 3, 2},
    {"mfma128x128_bk32_w2x2", 3, 3},
    {"mfma64x64_bk16_w2x2", 3, 4},
    {"mfma256x256_bk32_w2x4", 3, 5},
    {"mfma128x256_bk16_w2x2", 3, 6},
    {"mfma256x256_bk32_w2x4_direct", 3, 7},
    {"mfma256x256_bk16_w2x4_direct", 3, 8},
    {"mfma256x256_bk32_w4x2_direct", 3, 9},
    {"mfma256x256_bk32_w2x4_direct_swz32", 3, 10},
    {"mfma256x256_bk32_w2x4_direct_g4", 3, 11},
    {"mfma256x256_bk32_w2x4_direct_g16", 3, 12},
    {"mfma64x64_bk16_w2x2_k4", 3, 13},
    {"mfma64x64_bk32_w2x2_k4", 3, 14},
    {"mfma256x256_bk32_w2x4_direct_mi16", 3, 15},
    {"mfma256x256_bk32_w2x2_sched", 3, 16},
    {"mfma256x256_bk32_w2x2_sched_g4", 3, 17},
    {"mfma128x128_bk32_w2x2_sched", 3, 18},
    {"mfma128x128_bk32_w2x2_sched_g16", 3, 19},
    {"mfma64x64_bk32_w1x1_k4_sched", 3, 20},
    {"mfma16x16_w4_small", 3, 21},
    {"mfma32x32_w4_small", 3, 22},
    {"mfma16x16_w8_small", 3, 23},
    {"mfma96x96_bk16_w1x1_k4_sched", 3, 24},
    {"mfma64x64_bk32_w2x2_sched", 3, 25},
    {"mfma64x64_bk32_w2x2_4stage", 3, 26},
    {"mfma64x64_bk32_w2x2_2stage", 3, 27},
};
constexpr int kNumDiagnostics = (int)(sizeof(kDiagnostics) / sizeof(kDiagnostics[0]));

const char* const kRungNames[kNumRungs] = {
    "naive16x16", "tiled32_pad4", "regblock128x128_bk8_padA4", "mfma_auto"};

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 3u) != 0; }

// (rows - 1) * ld + cols must be addressable with 64-bit element offsets.
bool extent_fits(int64_t rows, int64_t cols, int64_t ld) {
    if (rows == 0 || cols == 0) return true;
    int64_t last;
    if (__builtin_mul_overflow(rows - 1, ld, &last)) return false;
    return !__builtin_add_overflow(last, cols, &last);
}

// op_a / op_b: 0 = the factor as stored, 1 = its transpose (A stored K x M,
// B stored N x K).
int validate(int op_a, int op_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             const float* B, int64_t ldb, const float* C, int64_t ldc) {
    if ((op_a != GEMM_F32_OP_N && op_a != GEMM_F32_OP_T) ||
        (op_b != GEMM_F32_OP_N && op_b != GEMM_F32_OP_T))
        return GEMM_F32_ERR_INVALID_OP;
    if (M < 0 || N < 0 || K < 0) return GEMM_F32_ERR_INVALID_DIM;
    const int64_t a_rows = op_a ? K : M, a_cols = op_a ? M : K;
    const int64_t b_rows = op_b ? N : K, b_cols = op_b ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return GEMM_F32_ERR_INVALID_LD;
    if (M == 0 || N == 0) return GEMM_F32_OK;           // nothing is read or written
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(C) || (K > 0 && (misaligned(A) || misaligned(B)))) return GEMM_F32_ERR_MISALIGNED;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_F32_ERR_TOO_LARGE;
    if (!extent_fits(a_rows, a_cols, lda) || !extent_fits(b_rows, b_cols, ldb) ||
        !extent_fits(M, N, ldc))
        return GEMM_F32_ERR_TOO_LARGE;
    // every launch uses at most one block per 16 x 16 outputs and at most 1024
    // threads per block; keep the grid below 2^32 work-items
    const int64_t blocks16 = ((M + 15) / 16) * ((N + 15) / 16);
    if (blocks16 > (int64_t)0xFFFFFFFF / 256) return GEMM_F32_ERR_TOO_LARGE;
    return GEMM_F32_OK;
}

int run(int rung, int config, int op_a, int op_b, int64_t M, int64_t N, int64_t K, const float* A,
        int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    const int st = validate(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc);
    if (st != GEMM_F32_OK) return st;
    if (M == 0 || N == 0) return GEMM_F32_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    GemmArgs p{(int)M, (int)N, (int)K, A, lda, B, ldb, C, ldc};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    switch (rung) {
        case 0: e = launch_naive(p, s); break;
        case 1: e = launch_tiled(p, s, config); break;
        case 2: e = launch_regblock(p, s, config); break;
        default:
            e = launch_mfma(p, s, config < 0 ? mfma_pick_config(p.M, p.N, p.K) : config, op_a, op_b);
            break;
    }
    if (e == hipErrorInvalidValue) return GEMM_F32_ERR_TOO_LARGE;
    if (e == hipErrorNotSupported) return GEMM_F32_ERR_INVALID_OP;
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

}  // namespace
}  // namespace gemmf32

using namespace gemmf32;

extern "C" int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                        const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    return run(3, -1, GEMM_F32_OP_N, GEMM_F32_OP_N, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int gemm_f32_op(int op_a, int op_b, int64_t M, int64_t N, int64_t K, const float* A,
                           int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                           void* stream) {
    return run(3, -1, op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int gemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K, const float* A,
                                int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                                void* stream) {
    if (variant >= 0 && variant < kNumRungs) {
        const int config = variant == 1 ? 4 : (variant == 2 ? 0 : -1);   // rung defaults
        return run(variant, config, GEMM_F32_OP_N, GEMM_F32_OP_N, M, N, K, A, lda, B, ldb, C, ldc,
                   stream);
    }
    const int d = variant - kDiagBase;
    if (d >= 0 && d < kNumDiagnostics)
        return run(kDiagnostics[d].rung, kDiagnostics[d].config, GEMM_F32_OP_N, GEMM_F32_OP_N, M, N,
                   K, A, lda, B, ldb, C, ldc, stream);
    return GEMM_F32_ERR_INVALID_VARIANT;
}

extern "C" int gemm_f32_num_variants(void) { return kNumRungs; }

extern "C" int gemm_f32_num_diagnostic_variants(void) { return kNumDiagnostics; }

extern "C" const char* gemm_f32_variant_name(int variant) {
    if (variant >= 0 && variant < kNumRungs) return kRungNames[variant];
    const int d = variant - kDiagBase;
    if (d >= 0 && d < kNumDiagnostics) return kDiagnostics[d].name;
    return nullptr;
}

extern "C" int gemm_f32_default_variant(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return -1;
    const int config = mfma_pick_config((int)M, (int)N, (int)K);
    for (int d = 0; d < kNumDiagnostics; ++d)
        if (kDiagnostics[d].rung == 3 && kDiagnostics[d].config == config) return kDiagBase + d;
    return -1;
}

extern "C" const char* gemm_f32_status_string(int status) {
    switch (status) {
        case GEMM_F32_OK: return "ok";
        case GEMM_F32_ERR_INVALID_DIM: return "invalid dimension: M, N and K must be >= 0";
        case GEMM_F32_ERR_INVALID_LD:
            return "invalid leading dimension: need lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N)";
        case GEMM_F32_ERR_NULL_PTR: return "null pointer for a non-empty matrix";
        case GEMM_F32_ERR_MISALIGNED: return "pointer not 4-byte aligned";
        case GEMM_F32_ERR_INVALID_VARIANT: return "unknown kernel variant";
        case GEMM_F32_ERR_TOO_LARGE: return "problem too large for the kernel index range or grid";
        case GEMM_F32_ERR_LAUNCH: return "kernel launch rejected by the HIP runtime";
        case GEMM_F32_ERR_DEVICE: return "no usable current HIP device";
        case GEMM_F32_ERR_INVALID_OP: return "invalid op: op_a and op_b must be GEMM_F32_OP_N or GEMM_F32_OP_T";
        case GEMM_F32_ERR_WORKSPACE: return "workspace smaller than reduce_sum_f32_workspace_size()";
        case GEMM_F32_ERR_INVALID_FORMAT: return "unknown 16-bit format: use GEMM_MIXED_BF16 or GEMM_MIXED_F16";
        case GEMM_F32_ERR_SCRATCH:
            return "partials exceed the library's fixed 1 MiB scratch: use reduce_sum_f32_variant with a workspace";
        default: return "unknown status";
    }
}

// A measurement helper: the vector-ALU FMA loop of probe.hip.
extern "C" int gemm_f32_valu_probe(int form, int64_t blocks, int iters, float* out, uint64_t* stamps,
                                   void* stream) {
    if (form < 0 || form > 2) return GEMM_F32_ERR_INVALID_VARIANT;
    if (blocks < 1 || iters < 0) return GEMM_F32_ERR_INVALID_DIM;
    if (blocks > 0x7FFFFFFF / 256) return GEMM_F32_ERR_TOO_LARGE;
    if (out == nullptr || stamps == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(out) || ((uintptr_t)stamps & 7u) != 0) return GEMM_F32_ERR_MISALIGNED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    const hipError_t e = launch_valu_probe(form, (int)blocks, iters, out, stamps, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// A measurement helper: the LDS read probe of probe.hip.
extern "C" int gemm_f32_lds_probe(int form, const int32_t* offsets, int iters, uint32_t* out, void* stream) {
    if (form < 0 || form > 3) return GEMM_F32_ERR_INVALID_VARIANT;
    if (iters < 0) return GEMM_F32_ERR_INVALID_DIM;
    if (offsets == nullptr || out == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(offsets) || misaligned(out)) return GEMM_F32_ERR_MISALIGNED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    const hipError_t e = launch_lds_probe(form, offsets, iters, out, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// A measurement helper: the copy-rate probe of probe.hip.
extern "C" int gemm_f32_copy_probe(int mode, int64_t blocks, int iters, const void* src, uint32_t* out,
                                   uint64_t* cycles, void* stream) {
    if (mode < 0 || mode > 1) return GEMM_F32_ERR_INVALID_VARIANT;
    if (blocks < 1 || iters < 0 || iters % 2 != 0) return GEMM_F32_ERR_INVALID_DIM;
    if (blocks > 0x7FFFFFFF / 256) return GEMM_F32_ERR_TOO_LARGE;
    if (src == nullptr || out == nullptr || cycles == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (((uintptr_t)src & 15u) != 0 || misaligned(out) || ((uintptr_t)cycles & 7u) != 0)
        return GEMM_F32_ERR_MISALIGNED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    const hipError_t e = launch_copy_probe(mode, (int)blocks, static_cast<const unsigned*>(src), iters, out, cycles,
                                           reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// A measurement helper: gemm_f32's k-split launch on the kernel's timeline
// instantiation (mfma_sched.hip).
extern "C" int gemm_f32_ksplit_timeline(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                                        const float* B, int64_t ldb, float* C, int64_t ldc, uint32_t* timeline,
                                        int64_t timeline_words, void* stream) {
    const int st = validate(GEMM_F32_OP_N, GEMM_F32_OP_N, M, N, K, A, lda, B, ldb, C, ldc);
    if (st != GEMM_F32_OK) return st;
    if (timeline == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(timeline)) return GEMM_F32_ERR_MISALIGNED;
    if (timeline_words < 32 || timeline_words % 32 != 0) return GEMM_F32_ERR_INVALID_DIM;
    GemmArgs p{(int)M, (int)N, (int)K, A, lda, B, ldb, C, ldc};
    if (M == 0 || N == 0 || !ksplit_f32_fits(p, GEMM_F32_OP_N, GEMM_F32_OP_N)) return GEMM_F32_ERR_INVALID_DIM;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    const int64_t blocks = timeline_words / 32;
    const hipError_t e = launch_ksplit_f32_timeline(p, reinterpret_cast<hipStream_t>(stream),
                                                    mfma_config_group_m(kMfmaKsplitConfig), timeline,
                                                    (int)(blocks < 0x7FFFFFFF ? blocks : 0x7FFFFFFF));
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// ---------------------------------------------------------------- transpose

namespace {
constexpr int kTransposeAuto = -1;

// The default transpose: 64 x 64 tiles with 128-bit accesses, handed out in
// diagonal order (with strides near a multiple of 4 KB, tiles handed out row
// by row make concurrent blocks touch addresses equal modulo a large power
// of two, the same HBM channels), with nontemporal stores and cacheable
// loads (variant 9): the output is written once and never read back, so
// keeping it out of the caches leaves them to the input.  Measured on nine
// shapes from 4096^2 to 16384^2 and rectangles, variant 9 was the fastest
// or within 3 % of it wherever the tile grid is square or the input holds
// 128 MiB or more; on a smaller rectangular input (8192 x 2048 with
// leading dimension 2056) the cached stores of variant 6 were 10 % faster.
int pick_transpose(int64_t rows, int64_t cols, int64_t /*ld_in*/, int64_t /*ld_out*/) {
    const bool square_grid = (rows + 63) / 64 == (cols + 63) / 64;
    const bool big = rows * cols * 4 >= ((int64_t)128 << 20);
    return (square_grid || big) ? 9 : 6;
}

int run_transpose(int variant, int64_t rows, int64_t cols, const float* in, int64_t ld_in, float* out,
                  int64_t ld_out, void* stream) {
    if (variant != kTransposeAuto && (variant < 0 || variant >= transpose_num_variants()))
        return GEMM_F32_ERR_INVALID_VARIANT;
    if (rows < 0 || cols < 0) return GEMM_F32_ERR_INVALID_DIM;
    if (ld_in < (cols > 1 ? cols : 1) || ld_out < (rows > 1 ? rows : 1)) return GEMM_F32_ERR_INVALID_LD;
    if (rows == 0 || cols == 0) return GEMM_F32_OK;
    if (in == nullptr || out == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(in) || misaligned(out)) return GEMM_F32_ERR_MISALIGNED;
    if (rows > INT_MAX || cols > INT_MAX || !extent_fits(rows, cols, ld_in) ||
        !extent_fits(cols, rows, ld_out))
        return GEMM_F32_ERR_TOO_LARGE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    if (variant == kTransposeAuto) variant = pick_transpose(rows, cols, ld_in, ld_out);
    const hipError_t e = launch_transpose(variant, (int)rows, (int)cols, in, ld_in, out, ld_out,
                                          reinterpret_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidValue) return GEMM_F32_ERR_TOO_LARGE;
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}
}  // namespace

extern "C" int transpose_f32_default_variant(int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out) {
    if (rows < 0 || cols < 0 || rows > INT_MAX || cols > INT_MAX) return -1;
    return pick_transpose(rows, cols, ld_in, ld_out);
}

extern "C" int transpose_f32(int64_t rows, int64_t cols, const float* in, int64_t ld_in, float* out,
                             int64_t ld_out, void* stream) {
    return run_transpose(kTransposeAuto, rows, cols, in, ld_in, out, ld_out, stream);
}

extern "C" int transpose_f32_variant(int variant, int64_t rows, int64_t cols, const float* in,
                                     int64_t ld_in, float* out, int64_t ld_out, void* stream) {
    return run_transpose(variant, rows, cols, in, ld_in, out, ld_out, stream);
}

extern "C" int transpose_f32_num_variants(void) { return transpose_num_variants(); }

extern "C" const char* transpose_f32_variant_name(int variant) {
    return transpose_variant_name(variant);
}

// ---------------------------------------------------------------- reduction

namespace {
constexpr int kReduceDefault = 4;

// Checks shared by the reduction entry points (no device needed).
int check_reduce(int variant, int64_t n, const float* x, const float* out) {
    if (variant < 0 || variant >= reduce_num_variants()) return GEMM_F32_ERR_INVALID_VARIANT;
    if (n < 0) return GEMM_F32_ERR_INVALID_DIM;
    if (out == nullptr || (n > 0 && x == nullptr)) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(out) || (n > 0 && misaligned(x))) return GEMM_F32_ERR_MISALIGNED;
    if (n > ((int64_t)1 << 39)) return GEMM_F32_ERR_TOO_LARGE;
    return GEMM_F32_OK;
}

int finish_reduce(hipError_t e) {
    if (e == hipErrorInvalidValue) return GEMM_F32_ERR_TOO_LARGE;
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

int run_reduce(int variant, int64_t n, const float* x, float* out, void* workspace, int64_t ws_bytes,
               void* stream) {
    const int st = check_reduce(variant, n, x, out);
    if (st != GEMM_F32_OK) return st;
    if (ws_bytes < 0) return GEMM_F32_ERR_INVALID_DIM;
    const int64_t need = 4 * reduce_workspace_floats(variant, n);
    if (ws_bytes < need) return GEMM_F32_ERR_WORKSPACE;
    if (need > 0 && workspace == nullptr) return GEMM_F32_ERR_NULL_PTR;
    if (need > 0 && misaligned(workspace)) return GEMM_F32_ERR_MISALIGNED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    return finish_reduce(launch_reduce(variant, n, x, out, static_cast<float*>(workspace),
                                       reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" int64_t reduce_sum_f32_workspace_size(int variant, int64_t n) {
    if (variant < 0 || variant >= reduce_num_variants() || n < 0) return -1;
    return 4 * reduce_workspace_floats(variant, n);
}

extern "C" int reduce_sum_f32(int64_t n, const float* x, float* out, void* workspace,
                              int64_t workspace_bytes, void* stream) {
    return run_reduce(kReduceDefault, n, x, out, workspace, workspace_bytes, stream);
}

extern "C" int reduce_sum_f32_variant(int variant, int64_t n, const float* x, float* out,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
    return run_reduce(variant, n, x, out, workspace, workspace_bytes, stream);
}

// The same reduction with the partials in the library's fixed per-device
// scratch instead of a caller's workspace: nothing is allocated, so callers
// that cannot allocate (stream capture, allocation-free loops) can use it.
extern "C" int reduce_sum_f32_variant_noalloc(int variant, int64_t n, const float* x, float* out,
                                              void* stream) {
    const int st = check_reduce(variant, n, x, out);
    if (st != GEMM_F32_OK) return st;
    if (reduce_workspace_floats(variant, n) > kReduceScratchFloats) return GEMM_F32_ERR_SCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    float* scratch = nullptr;
    if (reduce_scratch(dev, &scratch) != hipSuccess) return GEMM_F32_ERR_DEVICE;
    return finish_reduce(launch_reduce(variant, n, x, out, scratch, reinterpret_cast<hipStream_t>(stream)));
}

extern "C" int reduce_sum_f32_num_variants(void) { return reduce_num_variants(); }

extern "C" const char* reduce_sum_f32_variant_name(int variant) { return reduce_variant_name(variant); }

// ---------------------------------------------------------- mixed precision

namespace {
constexpr int kMixedAuto = -1;

bool misaligned2(const void* ptr) { return ((uintptr_t)ptr & 1u) != 0; }

// config: a gemm_mixed variant (kMixedAuto: picked for the shape); with a
// transposed factor (op_a or op_b = 1) only kMixedAuto, on the op kernels.
int run_mixed(int config, int op_a, int op_b, int format, int64_t M, int64_t N, int64_t K,
              const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
              void* stream) {
    if ((op_a != GEMM_F32_OP_N && op_a != GEMM_F32_OP_T) || (op_b != GEMM_F32_OP_N && op_b != GEMM_F32_OP_T))
        return GEMM_F32_ERR_INVALID_OP;
    if (config != kMixedAuto && (config < 0 || config >= mixed_num_configs()))
        return GEMM_F32_ERR_INVALID_VARIANT;
    if (format != GEMM_MIXED_BF16 && format != GEMM_MIXED_F16) return GEMM_F32_ERR_INVALID_FORMAT;
    if (M < 0 || N < 0 || K < 0) return GEMM_F32_ERR_INVALID_DIM;
    const int64_t a_rows = op_a ? K : M, a_cols = op_a ? M : K;
    const int64_t b_rows = op_b ? N : K, b_cols = op_b ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return GEMM_F32_ERR_INVALID_LD;
    if (M == 0 || N == 0) return GEMM_F32_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return GEMM_F32_ERR_NULL_PTR;
    if (misaligned(C) || (K > 0 && (misaligned2(A) || misaligned2(B)))) return GEMM_F32_ERR_MISALIGNED;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_F32_ERR_TOO_LARGE;
    if (!extent_fits(a_rows, a_cols, lda) || !extent_fits(b_rows, b_cols, ldb) || !extent_fits(M, N, ldc))
        return GEMM_F32_ERR_TOO_LARGE;
    const int64_t blocks16 = ((M + 15) / 16) * ((N + 15) / 16);
    if (blocks16 > (int64_t)0xFFFFFFFF / 256) return GEMM_F32_ERR_TOO_LARGE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_F32_ERR_DEVICE;
    const Gemm16Args p{(int)M, (int)N, (int)K, A, lda, B, ldb, C, ldc};
    hipError_t e;
    if (op_a || op_b) {
        e = launch_mixed_op(p, reinterpret_cast<hipStream_t>(stream), format, op_a, op_b);
    } else {
        if (config == kMixedAuto) config = mixed_pick_config(p.M, p.N, p.K);
        e = launch_mixed(p, reinterpret_cast<hipStream_t>(stream), format, config);
    }
    if (e == hipErrorInvalidValue) return GEMM_F32_ERR_TOO_LARGE;
    return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}
}  // namespace

extern "C" int gemm_mixed(int format, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    return run_mixed(kMixedAuto, GEMM_F32_OP_N, GEMM_F32_OP_N, format, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int gemm_mixed_op(int op_a, int op_b, int format, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                             int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    return run_mixed(kMixedAuto, op_a, op_b, format, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int gemm_mixed_variant(int variant, int format, int64_t M, int64_t N, int64_t K,
                                  const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                  float* C, int64_t ldc, void* stream) {
    return run_mixed(variant, GEMM_F32_OP_N, GEMM_F32_OP_N, format, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

extern "C" int gemm_mixed_num_variants(void) { return mixed_num_configs(); }

extern "C" const char* gemm_mixed_variant_name(int variant) { return mixed_config_name(variant); }

extern "C" int gemm_mixed_default_variant(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return -1;
    return mixed_pick_config((int)M, (int)N, (int)K);
}
