// small.hip -- rung 3 for products too small to fill the chip with tiles.
//
// The tiled product of the pages' shared-memory chapter (PMPP chapter 5
// notes, sections 5.4-5.5) gives each block one output tile and runs its
// phases one after another.  With few output elements (a 256 x 256 product
// has 16 tiles of 64 x 64 for 256 compute units) the time goes to latency
// -- the first loads, the chain of phases, the final store -- not to
// arithmetic, so here the output tiles are small (16 x 16 or 32 x 32, one
// block each: a 256 x 256 product has 256 blocks) and the K extent of each
// tile is split over the W waves of its block: wave w takes the 16-deep k
// groups w, w + W, w + 2W, ...  No operand is shared between the lanes of a
// wave inside one matrix instruction's k group, so each lane loads its own
// operands straight from global memory into registers (ghost elements
// outside the matrices are zeros, as in the pages' tiled kernel), four
// groups in flight per wave; the partial tiles of the W waves then meet in
// LDS and are added in wave order (deterministic; the same bits for every op
// pair), and the guarded store writes the tile.
//
// Matrix instruction: v_mfma_f32_16x16x4_f32 (16 x 16 block, k = 4): lane l
// supplies A[l % 16][l / 16] and B[l / 16][l % 16], accumulator register r
// holds D[4 (l / 16) + r][l % 16].  Within a group of 16 k at kg, lane group
// g = l / 16 feeds k = kg + 4 g + s to the s-th of four instructions, so a
// lane's four values of a factor are four consecutive k of one row or
// column: one 128-bit load when the factor is stored k-contiguous (A as
// stored, B stored transposed), four 32-bit loads, each coalesced over 16
// consecutive columns, when it is stored mn-contiguous.
#include "launch.h"

namespace gemmf32 {

namespace {

constexpr int kGroupK = 16;           // k values per group of four instructions
constexpr int kInFlight = 4;          // groups whose operands a wave has in flight

// Values (mn, k .. k + 3) of a factor of extent `ext` along mn and K along k,
// zeros outside: stored k-contiguous (element (mn, k) at X[mn * ld + k]) or
// mn-contiguous (at X[k * ld + mn]).
template <bool KC>
__device__ __forceinline__ floatx4 fetch4(const float* __restrict__ X, int64_t ld, int mn, int ext, int k, int K) {
    if constexpr (KC) {
        return load4_ghost(X, mn, ext, k, K, ld);
    } else {
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (mn < ext) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (k + s < K) v[s] = X[(int64_t)(k + s) * ld + mn];
        }
        return v;
    }
}

// FM x FN blocks of 16 x 16 per tile, W waves splitting its k groups.
template <int FM, int FN, int W, bool KCA, bool KCB>
__global__ __launch_bounds__(64 * W)
void gemm_f32_small_kernel(GemmArgs p, int tiles_n) {
    constexpr int BM = 16 * FM, BN = 16 * FN;
    constexpr int PART = FM * FN * 256;                 // one wave's partial tile, in floats
    __shared__ __attribute__((aligned(16))) float part[W * PART];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mn = lane & 15, g = lane >> 4;

    const int tiles = (int)gridDim.x;
    const int logical = xcd_contiguous((int)blockIdx.x, tiles);
    const int m0 = (logical / tiles_n) * BM;
    const int n0 = (logical % tiles_n) * BN;

    const int groups = ceil_div(p.K, kGroupK);
    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Operands of this wave's local group u (group w + W u), into slot t.
    floatx4 fa[kInFlight][FM], fb[kInFlight][FN];
    auto fetch = [&](int t, int u) __attribute__((always_inline)) {
        const int k = (w + W * u) * kGroupK + 4 * g;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[t][i] = fetch4<KCA>(p.A, p.lda, m0 + 16 * i + mn, p.M, k, p.K);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[t][j] = fetch4<KCB>(p.B, p.ldb, n0 + 16 * j + mn, p.N, k, p.K);
    };
    const int mine = groups > w ? (groups - 1 - w) / W + 1 : 0;   // this wave's groups (uniform)
#pragma unroll
    for (int t = 0; t < kInFlight; ++t)
        if (t < mine) fetch(t, t);
    for (int base = 0; base < mine; base += kInFlight) {
#pragma unroll
        for (int t = 0; t < kInFlight; ++t) {
            if (base + t >= mine) break;
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[t][i][s], fb[t][j][s], acc[i][j], 0, 0, 0);
            if (base + t + kInFlight < mine) fetch(t, base + t + kInFlight);
        }
    }

    // Partial tiles: register r of block (i, j) of lane l of wave v at
    // v PART + ((i FN + j) 4 + r) 64 + l.  Output (row, col) of the tile is
    // block (row / 16, col / 16), lane 16 ((row % 16) / 4) + col % 16,
    // register row % 4.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[w * PART + ((i * FN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int o = tid; o < BM * BN; o += 64 * W) {
        const int row = o / BN, col = o % BN;
        const int rr = row & 15, cc = col & 15;
        const int at = (((row >> 4) * FN + (col >> 4)) * 4 + (rr & 3)) * 64 + 16 * (rr >> 2) + cc;
        float v = part[at];
#pragma unroll
        for (int u = 1; u < W; ++u) v += part[u * PART + at];
        if (m0 + row < p.M && n0 + col < p.N) p.C[(int64_t)(m0 + row) * p.ldc + n0 + col] = v;
    }
}

template <int FM, int FN, int W, bool KCA, bool KCB>
hipError_t launch_small_kernel(const GemmArgs& p, hipStream_t s) {
    const int tiles_m = ceil_div(p.M, 16 * FM), tiles_n = ceil_div(p.N, 16 * FN);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_f32_small_kernel<FM, FN, W, KCA, KCB>), dim3((unsigned)blocks), dim3(64 * W), 0, s,
                       p, tiles_n);
    return hipGetLastError();
}

template <int FM, int FN, int W>
hipError_t launch_small_ops(const GemmArgs& p, hipStream_t s, int op_a, int op_b) {
    switch (2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_small_kernel<FM, FN, W, true, false>(p, s);
        case 1: return launch_small_kernel<FM, FN, W, true, true>(p, s);
        case 2: return launch_small_kernel<FM, FN, W, false, false>(p, s);
        default: return launch_small_kernel<FM, FN, W, false, true>(p, s);
    }
}

}  // namespace

// shape: 0 = 16 x 16 tiles on 4 waves, 1 = 32 x 32 tiles on 4 waves,
// 2 = 16 x 16 tiles on 8 waves.
hipError_t launch_small_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int shape) {
    switch (shape) {
        case 0: return launch_small_ops<1, 1, 4>(p, s, op_a, op_b);
        case 1: return launch_small_ops<2, 2, 4>(p, s, op_a, op_b);
        default: return launch_small_ops<1, 1, 8>(p, s, op_a, op_b);
    }
}

}  // namespace gemmf32
