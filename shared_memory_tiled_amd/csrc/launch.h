// launch.h -- host-side declarations of the kernel launchers and their
// configuration tables, shared by the kernel translation units and api.hip
// (not part of the public interface).  Device code lives in the .hip files and
// in gemm_internal.h.
#pragma once

#include "gemm_internal.h"

namespace gemmf32 {

// Launchers (asynchronous; return the launch status of the HIP runtime).
hipError_t launch_naive(const GemmArgs& p, hipStream_t s);
hipError_t launch_tiled(const GemmArgs& p, hipStream_t s, int pad);
hipError_t launch_regblock(const GemmArgs& p, hipStream_t s, int config);
hipError_t launch_mfma(const GemmArgs& p, hipStream_t s, int config, int op_a, int op_b);

// Shared-tile transpose (transpose.hip): out (cols x rows) = in^T.
hipError_t launch_transpose(int variant, int rows, int cols, const float* in, int64_t ld_in,
                            float* out, int64_t ld_out, hipStream_t s);
int transpose_num_variants();
const char* transpose_variant_name(int v);

// Mixed-precision product (mfma16.hip): C (binary32) = A x B with A and B
// holding 16-bit patterns of one format (0 bfloat16, 1 binary16), row-major,
// leading dimensions in elements.  Validated like GemmArgs.
struct Gemm16Args {
    int M, N, K;
    const uint16_t* A; int64_t lda;
    const uint16_t* B; int64_t ldb;
    float* C; int64_t ldc;
};
hipError_t launch_mixed(const Gemm16Args& p, hipStream_t s, int format, int config);
int mixed_num_configs();
const char* mixed_config_name(int config);
int mixed_pick_config(int M, int N, int K);
// op(A) x op(B) with either factor stored transposed (op 1): A stored K x M,
// B stored N x K; validated like GemmArgs with the leading dimensions of the
// stored matrices.
hipError_t launch_mixed_op(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b);
// 16-bit product on 64 x 64 tiles whose four waves split the phases
// (mfma16_ksplit.hip): whether it takes the problem (K a multiple of 8, an
// mn-contiguous factor's width even, vector-aligned operands below 2^31
// bytes), and its launcher (format 0 bfloat16, 1 binary16; op 1: that factor
// stored transposed).
bool ksplit16_fits(const Gemm16Args& p, int op_a, int op_b);
hipError_t launch_ksplit16(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b);
// The same split on 128 x 128 tiles, for a few hundred of them
// (mfma16_ksplit128.hip): whether it takes the problem (as above), and its
// launcher, with tile-row groups of group_m.
bool ksplit128_fits(const Gemm16Args& p, int op_a, int op_b);
hipError_t launch_ksplit128(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m);
// The scheduled 256 x 256 kernel on the 16 x 16 x 32 instruction
// (mfma16_wide.hip): whether it takes the problem (those of the 32 x 32 x 16
// scheduled kernel, with any even K), and its launcher (the caller checks),
// with tile-row groups of group_m.
bool wide_fits(const Gemm16Args& p, int op_a, int op_b);
hipError_t launch_wide16(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m);
// The same kernel on 192 x 192 tiles (each wave 96 x 96) or 160 x 160 tiles
// (80 x 80), for problems whose 256 x 256 tiles fill the CUs' rounds badly;
// the same problems fit.
hipError_t launch_wide16_192(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m);
hipError_t launch_wide16_160(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m);
// The same product with four 32-deep LDS stages (mfma16_wide4.hip), as
// stored (A k-contiguous, B mn-contiguous) only.
hipError_t launch_wide16_4stage(const Gemm16Args& p, hipStream_t s, int format, int group_m);

// Sum reduction (reduce.hip): *out = sum of x[0 .. n-1].
hipError_t launch_reduce(int variant, int64_t n, const float* x, float* out, float* ws, hipStream_t s);
int64_t reduce_workspace_floats(int variant, int64_t n);
// The fixed per-device scratch (reduce.hip) that takes the partials of the
// entry point for callers that cannot allocate: its size in floats, and its
// address on `device` (looked up once per device; the device must be
// current on the first call for it).
constexpr int64_t kReduceScratchFloats = (int64_t)1 << 18;     // 1 MiB
hipError_t reduce_scratch(int device, float** ptr);
int reduce_num_variants();
const char* reduce_variant_name(int v);

// Number of MFMA / register-blocked tile configurations and their names.
int mfma_num_configs();
const char* mfma_config_name(int config);
int mfma_pick_config(int M, int N, int K);
// Four-wave kernel with an explicit instruction order (mfma_sched.hip) on
// 256 x 256 or 128 x 128 tiles: whether it takes the problem (K, M and N
// multiples of 4, stored factors below 2^31 bytes), and its launcher
// (op 1: factor stored transposed; tile 256 or 128).
bool sched_f32_fits(const GemmArgs& p, int op_a, int op_b);
hipError_t launch_sched_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m, int tile);
// 64 x 64 tiles of 2 x 2 waves of one 32 x 32 block each, from `stages`
// (2 or 4) LDS stages (mfma_sched.hip); the problems sched_f32_fits takes.
hipError_t launch_tile64_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m, int stages);
// Four waves splitting the phases of one 64 x 64 tile (mfma_sched.hip):
// whether it takes the problem (K, M and N multiples of 4, stored factors
// below 2^31 bytes), and its launcher.
bool ksplit_f32_fits(const GemmArgs& p, int op_a, int op_b);
hipError_t launch_ksplit_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m);
// Four waves splitting the phases of one 96 x 96 tile (mfma_ksplit96.hip):
// whether it takes the problem (K, M and N multiples of 4, stored factors
// below 2^31 bytes), and its launcher.
bool ksplit96_f32_fits(const GemmArgs& p, int op_a, int op_b);
hipError_t launch_ksplit96_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m);
// Measurement helper: the same launch (factors as stored) on the kernel's
// timeline instantiation, which also writes 8 words per wave of the first
// timeline_blocks blocks to `timeline`.
hipError_t launch_ksplit_f32_timeline(const GemmArgs& p, hipStream_t s, int group_m, uint32_t* timeline,
                                      int timeline_blocks);
// The tile-group height a configuration of launch_mfma launches with, and
// the configuration gemm_f32 runs the k-split kernel as.
int mfma_config_group_m(int config);
constexpr int kMfmaKsplitConfig = 20;
// Small products (small.hip): 16 x 16 or 32 x 32 output tiles whose k
// groups are split over the waves of each block, operands loaded straight
// into registers (shape 0: 16 x 16 on 4 waves, 1: 32 x 32 on 4 waves, 2: 16
// x 16 on 8 waves).  Any sizes, leading dimensions and op pair.
hipError_t launch_small_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int shape);
// Measurement helper (probe.hip): a loop of non-packed fp32 FMAs on the
// vector ALU in operand form `form` (0 scalar-register operand, 1 vector
// registers, 2 8 x 8 outer product), `blocks` blocks of 256 threads.
hipError_t launch_valu_probe(int form, int blocks, int iters, float* out, uint64_t* stamps, hipStream_t s);
// Measurement helper (probe.hip): one wave reading LDS at 64 given byte
// offsets, `iters` times (form 0 ds_read_b32, 1 ds_read_b64, 2
// ds_read_b128, 3 ds_read_b64_tr_b16).
hipError_t launch_lds_probe(int form, const int* offs, int iters, unsigned* out, hipStream_t s);
// Measurement helper (probe.hip): 1 KB wave loads from an L2-resident
// buffer, into LDS (mode 0) or vector registers (mode 1); `blocks` blocks of
// 4 waves, each block reading its own 64 KB of src.
hipError_t launch_copy_probe(int mode, int blocks, const unsigned* src, int iters, unsigned* out, uint64_t* cycles,
                             hipStream_t s);
int regblock_num_configs();
const char* regblock_config_name(int config);

}  // namespace gemmf32
