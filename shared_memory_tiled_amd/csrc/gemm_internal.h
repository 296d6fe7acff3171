// gemm_internal.h -- definitions shared by the kernel translation units of the
// gfx950 fp32 GEMM library (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmf32 {

// One product C = A x B on row-major binary32 matrices (see gemm_f32.h).
// Sizes were validated by the entry point: 0 < M, N < 2^31, 0 <= K < 2^31.
// For the MFMA kernels A and/or B may be stored transposed (see mfma.hip);
// the other kernels take them as stored.
struct GemmArgs {
    int M, N, K;
    const float* A; int64_t lda;
    const float* B; int64_t ldb;
    float* C; int64_t ldc;
};

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__host__ __device__ constexpr int ceil_div(int a, int b) { return (int)(((int64_t)a + b - 1) / b); }

// gfx950 deals consecutive workgroups to its eight XCDs in turn, and each XCD
// has its own L2.  This maps block b to a logical tile index so that each XCD
// walks one contiguous run of the nblocks tiles.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int b, int nblocks) {
    const int per = nblocks / kXcds, extra = nblocks % kXcds;
    const int x = b % kXcds, local = b / kXcds;
    return x * per + min(x, extra) + local;
}

// Four consecutive floats of row `r` starting at column `c` of a row-major
// matrix with `rows` x `cols` valid entries and leading dimension `ld`.
// Slots outside the matrix read as +0 (ghost elements) and are never loaded.
// The in-range case is one 128-bit load; the pointer only needs 4-byte
// alignment (gfx9 runs global memory in unaligned-access mode, so a dword
// aligned dwordx4 load is legal), which lets offset sub-matrix views use it.
__device__ __forceinline__ floatx4 load4_ghost(const float* __restrict__ base, int r, int rows,
                                               int c, int cols, int64_t ld) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < rows) {
        const float* p = base + (int64_t)r * ld + c;
        if (c + 3 < cols) {
            __builtin_memcpy(&v, p, 16);
        } else {
            if (c + 0 < cols) v[0] = p[0];
            if (c + 1 < cols) v[1] = p[1];
            if (c + 2 < cols) v[2] = p[2];
        }
    }
    return v;
}

// Stores up to four consecutive outputs of row `r` from column `c`, skipping
// anything outside the rows x cols window (the guarded final store).
__device__ __forceinline__ void store4_guarded(float* __restrict__ base, int r, int rows, int c,
                                               int cols, int64_t ld, floatx4 v) {
    if (r >= rows) return;
    float* p = base + (int64_t)r * ld + c;
    if (c + 3 < cols) {
        __builtin_memcpy(p, &v, 16);
    } else {
        if (c + 0 < cols) p[0] = v[0];
        if (c + 1 < cols) p[1] = v[1];
        if (c + 2 < cols) p[2] = v[2];
    }
}

}  // namespace gemmf32
