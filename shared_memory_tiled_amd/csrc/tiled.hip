// tiled.hip -- rung 1: the shared-memory (LDS) tiled product with T = 32.
//
// Follows the tiled kernel of the pages: "03 CUDA Shared Memory: Tiling, Bank
// Conflicts, and Reduction", section "Shared Memory와 Tiling" (T = 32, one
// output per thread, a T x T tile of A and of B copied cooperatively per
// phase, two barriers per phase), with the ghost-element treatment of the
// PMPP chapter 5 notes "메모리 계층과 데이터 지역성", sections 5.4-5.5
// (ceil(K/T) phases, out-of-range tile slots set to zero, only the final
// store range checked, no thread leaves before the last barrier).
//
// What changes for gfx950:
//  * Cooperative copy with 128-bit loads.  A 32 x 32 tile is 256 float4
//    chunks; waves 0-3 copy the A tile and waves 4-7 the B tile (a
//    wave-uniform role, so no divergence), each lane one row-contiguous
//    chunk.  A wave's 64 chunks cover eight whole 128-byte tile rows.
//  * Padded rows.  A wave64 spans two rows (ty, ty+1) of the 32 x 32 block,
//    so the A-tile read As[ty][k] touches two words ROW_STRIDE apart rather
//    than the single broadcast word of a 32-lane warp.  Rows are padded by
//    PAD words; PAD = 4 keeps each row 16-byte aligned for the 128-bit LDS
//    stores.  PAD = 0 and PAD = 1 are built as diagnostic variants so that
//    the LDS bank-conflict counter can compare the layouts.
#include "launch.h"

namespace gemmf32 {

template <int PAD>
__global__ __launch_bounds__(1024) void gemm_tiled32_kernel(GemmArgs p, int tiles_n) {
    constexpr int T = 32;
    constexpr int ROW_STRIDE = T + PAD;
    __shared__ float As[T * ROW_STRIDE];
    __shared__ float Bs[T * ROW_STRIDE];

    const int tx = threadIdx.x, ty = threadIdx.y;          // block is 32 x 32
    const int tid = ty * T + tx;
    const int row0 = (int)(blockIdx.x / tiles_n) * T;
    const int col0 = (int)(blockIdx.x % tiles_n) * T;
    const int row = row0 + ty, col = col0 + tx;

    // Copy role of this thread: chunk q of the A tile (tid < 256) or of the B
    // tile (256 <= tid < 512); chunk q is row q / 8, columns 4 (q % 8) .. +3.
    const int q = tid & 255;
    const int cr = q >> 3, cc = (q & 7) << 2;

    float acc = 0.0f;
    const int phases = ceil_div(p.K, T);
    for (int ph = 0; ph < phases; ++ph) {
        const int k0 = ph * T;
        if (tid < 256) {
            floatx4 v = load4_ghost(p.A, row0 + cr, p.M, k0 + cc, p.K, p.lda);
            float* dst = &As[cr * ROW_STRIDE + cc];
            dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
        } else if (tid < 512) {
            floatx4 v = load4_ghost(p.B, k0 + cr, p.K, col0 + cc, p.N, p.ldb);
            float* dst = &Bs[cr * ROW_STRIDE + cc];
            dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
        }
        __syncthreads();          // barrier 1: both tiles are complete
#pragma unroll
        for (int k = 0; k < T; ++k)
            acc = fmaf(As[ty * ROW_STRIDE + k], Bs[k * ROW_STRIDE + tx], acc);
        __syncthreads();          // barrier 2: nobody still reads this phase's tiles
    }
    if (row < p.M && col < p.N)
        p.C[(int64_t)row * p.ldc + col] = acc;
}

hipError_t launch_tiled(const GemmArgs& p, hipStream_t s, int pad) {
    const int tiles_n = ceil_div(p.N, 32);
    const unsigned blocks = (unsigned)tiles_n * (unsigned)ceil_div(p.M, 32);
    const dim3 block(32, 32);
    switch (pad) {
        case 0: hipLaunchKernelGGL(gemm_tiled32_kernel<0>, dim3(blocks), block, 0, s, p, tiles_n); break;
        case 1: hipLaunchKernelGGL(gemm_tiled32_kernel<1>, dim3(blocks), block, 0, s, p, tiles_n); break;
        default: hipLaunchKernelGGL(gemm_tiled32_kernel<4>, dim3(blocks), block, 0, s, p, tiles_n); break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
