// regblock.hip -- rung 2: register-blocked, double-buffered tiled product.
//
// The pages name the next steps after a square tile: a thread keeps several
// outputs in registers and accumulates them there (first page, "Occupancy와
// Block 크기", register tiling; PMPP one-volume notes, "Thread Coarsening"),
// and the tile pipeline is double buffered (first page's reading list, the
// threadblock / thread tiling with register reuse and double buffering line).
// The phase loop, ghost zeros and guarded store are those of the tiled
// kernel (PMPP chapter 5 notes, sections 5.4-5.5).
//
// Layout on gfx950:
//  * workgroup tile 128 x 128, phase depth BK, 256 threads (four waves);
//    thread (ty, tx) = (tid / 16, tid % 16) owns the 8 x 8 outputs at rows
//    {4 ty .. 4 ty + 3, 64 + 4 ty .. +3} and columns {4 tx .. +3, 64 + 4 tx ..
//    +3} -- two 4-wide groups per side so that every LDS read is one 128-bit
//    read and a wave's B read is 256 contiguous bytes.
//  * the A tile is stored k-major (transposed while it is written to LDS) so
//    that a thread's four A operands for one k are contiguous; rows are padded
//    by PAD_A words.  With PAD_A = 4 the two k rows written by one 32-lane
//    half of a wave land 16 banks apart instead of on the same banks.
//  * two LDS buffers: the next phase's tile is loaded from global memory into
//    registers before the current phase's inner products and written to the
//    other buffer after them, so one barrier per phase orders both the write
//    before the next read and the reads before the overwrite two phases on.
//  * per k step a thread reads 16 floats from LDS for 64 fused multiply-adds
//    (1 byte of LDS per FMA), each a v_fmac_f32 with all three operands in
//    vector registers.  Packed FP32 is disabled for this library; on gfx950
//    the non-packed form with vector-register operands still issues one
//    wave64 FMA per SIMD every two cycles (measured: 0.43 per cycle at 8
//    waves per SIMD, where a form with a scalar-register operand reaches
//    only half that), so the VALU ceiling of this rung is the chip's fp32
//    peak, 256 FLOP per clock per CU.
#include "launch.h"

namespace gemmf32 {

template <int BK, int PAD_A, int PAD_B>
__global__ __launch_bounds__(256) void gemm_regblock_kernel(GemmArgs p, int tiles_n) {
    constexpr int BM = 128, BN = 128;
    constexpr int SA = BM + PAD_A;           // k-major A rows
    constexpr int SB = BN + PAD_B;           // k-major B rows
    constexpr int A_CHUNKS = BM * BK / 4 / 256;   // float4 chunks per thread
    constexpr int B_CHUNKS = BN * BK / 4 / 256;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for 256 threads");
    __shared__ __attribute__((aligned(16))) float As[2][BK * SA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];

    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int m0 = (int)(blockIdx.x / tiles_n) * BM;
    const int n0 = (int)(blockIdx.x % tiles_n) * BN;

    floatx4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * 256;                 // chunk: row q / (BK/4)
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
            ra[u] = load4_ghost(p.A, m0 + r, p.M, k0 + c, p.K, p.lda);
        }
#pragma unroll
        for (int u = 0; u < B_CHUNKS; ++u) {
            const int q = tid + u * 256;                 // chunk: row q / (BN/4)
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            rb[u] = load4_ghost(p.B, k0 + r, p.K, n0 + c, p.N, p.ldb);
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * 256;
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) As[buf][(c + e) * SA + r] = ra[u][e];
        }
#pragma unroll
        for (int u = 0; u < B_CHUNKS; ++u) {
            const int q = tid + u * 256;
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            *reinterpret_cast<floatx4*>(&Bs[buf][r * SB + c]) = rb[u];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const int phases = ceil_div(p.K, BK);
    if (phases > 0) {
        load_tiles(0);
        store_tiles(0);
    }
    __syncthreads();
    for (int ph = 0; ph < phases; ++ph) {
        const int cur = ph & 1;
        const bool more = ph + 1 < phases;
        if (more) load_tiles((ph + 1) * BK);     // in flight during the math below
        const float* __restrict__ as = As[cur];
        const float* __restrict__ bs = Bs[cur];
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const floatx4 a0 = *reinterpret_cast<const floatx4*>(&as[k * SA + 4 * ty]);
            const floatx4 a1 = *reinterpret_cast<const floatx4*>(&as[k * SA + 64 + 4 * ty]);
            const floatx4 b0 = *reinterpret_cast<const floatx4*>(&bs[k * SB + 4 * tx]);
            const floatx4 b1 = *reinterpret_cast<const floatx4*>(&bs[k * SB + 64 + 4 * tx]);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) store_tiles(cur ^ 1);
        __syncthreads();        // one barrier per phase (two LDS buffers)
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
        const floatx4 lo = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        const floatx4 hi = {acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
        store4_guarded(p.C, row, p.M, n0 + 4 * tx, p.N, p.ldc, lo);
        store4_guarded(p.C, row, p.M, n0 + 64 + 4 * tx, p.N, p.ldc, hi);
    }
}

namespace {
struct RegblockConfig { const char* name; };
const RegblockConfig kRegblockConfigs[] = {
    {"regblock128x128_bk8_padA4"},     // the rung
    {"regblock128x128_bk8_padA0"},     // diagnostic: unpadded A tile
    {"regblock128x128_bk16_padA4"},    // diagnostic: deeper phases
};
}  // namespace

int regblock_num_configs() { return (int)(sizeof(kRegblockConfigs) / sizeof(kRegblockConfigs[0])); }
const char* regblock_config_name(int c) {
    return (c >= 0 && c < regblock_num_configs()) ? kRegblockConfigs[c].name : nullptr;
}

hipError_t launch_regblock(const GemmArgs& p, hipStream_t s, int config) {
    const int tiles_n = ceil_div(p.N, 128);
    const unsigned blocks = (unsigned)tiles_n * (unsigned)ceil_div(p.M, 128);
    switch (config) {
        case 1: hipLaunchKernelGGL((gemm_regblock_kernel<8, 0, 4>), dim3(blocks), dim3(256), 0, s, p, tiles_n); break;
        case 2: hipLaunchKernelGGL((gemm_regblock_kernel<16, 4, 4>), dim3(blocks), dim3(256), 0, s, p, tiles_n); break;
        default: hipLaunchKernelGGL((gemm_regblock_kernel<8, 4, 4>), dim3(blocks), dim3(256), 0, s, p, tiles_n); break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
