// naive.hip -- rung 0: one thread per output element, operands straight from
// global memory.
//
// Follows the naive matrix product of the first page ("03 CUDA Shared
// Memory: Tiling, Bank Conflicts, and Reduction", section "Shared Memory와
// Tiling") and the guarded form with 16 x 16 blocks and a grid of
// ceil(W/16) x ceil(H/16) from the PMPP one-volume notes ("PMPP 단권화", the
// naive matrix-product baseline and its launch configuration).  Each k step
// reads one A and one B float for one multiply-add: 0.25 FLOP per byte of
// global reads, the bound the PMPP chapter 5 notes (section 5.1) derive.
//
// On wave64 a 16 x 16 workgroup is four waves, each covering four rows of
// sixteen outputs: the B read of a wave is four copies of 16 consecutive
// floats and the A read is four broadcast addresses.
#include "launch.h"

namespace gemmf32 {

// The ceil(N/16) x ceil(M/16) blocks are numbered along one grid dimension
// (block b is tile column b % tiles_n, tile row b / tiles_n), which keeps the
// launch within the grid limits for any matrix that fits in memory.
__global__ __launch_bounds__(256) void gemm_naive_kernel(GemmArgs p, int tiles_n) {
    const int col = (int)(blockIdx.x % tiles_n) * 16 + threadIdx.x;
    const int row = (int)(blockIdx.x / tiles_n) * 16 + threadIdx.y;
    // This kernel has no barrier, so out-of-range threads may leave early.
    if (row >= p.M || col >= p.N) return;
    const float* __restrict__ a = p.A + (int64_t)row * p.lda;
    const float* __restrict__ b = p.B + col;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k)
        acc = fmaf(a[k], b[(int64_t)k * p.ldb], acc);
    p.C[(int64_t)row * p.ldc + col] = acc;
}

hipError_t launch_naive(const GemmArgs& p, hipStream_t s) {
    const int tiles_n = ceil_div(p.N, 16);
    const unsigned blocks = (unsigned)tiles_n * (unsigned)ceil_div(p.M, 16);
    hipLaunchKernelGGL(gemm_naive_kernel, dim3(blocks), dim3(16, 16), 0, s, p, tiles_n);
    return hipGetLastError();
}

}  // namespace gemmf32
