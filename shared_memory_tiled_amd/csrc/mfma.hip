// mfma.hip -- rung 3: the tiled product on the CDNA4 matrix cores.
//
// Same phase structure as the pages' tiled kernel (PMPP chapter 5 notes
// "메모리 계층과 데이터 지역성", sections 5.4-5.5: cooperative copies of an A
// and a B tile per phase, ghost zeros past the edges, guarded final store),
// with register tiling and double buffering as in rung 2, and the
// multiply-adds of a phase done by v_mfma_f32_32x32x2_f32 instead of VALU
// FMAs.  The pages use matrix units only with 16-bit inputs (PMPP one-volume
// notes, deep-learning chapter: the FC layer is a GEMM on tensor cores); the
// fp32 matrix instruction is this library's reading for an fp32 product.
//
// v_mfma_f32_32x32x2_f32: D(32x32) += A(32x2) B(2x32) per wave, 16 passes.
// Lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator
// register r of lane l holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// The order of the k terms inside a phase is free (the sum is the same up
// to rounding), so for each group of 8 k values lane half h = l / 32 feeds
// k = kg + 4h + s to the s-th of four instructions.  A lane's four A
// operands are then contiguous and come from LDS in one 128-bit read.
//
// LDS layout per stage (two stages, one barrier per phase):
//   A: BM rows x BK k, m-major as in global memory, row stride SA = BK + 4.
//      One 128-bit read per lane walks down a column group of the tile; with
//      the stride 4 words off a multiple of 32 banks, eight consecutive
//      rows fall on distinct 4-bank groups (the first page's padding rule,
//      "Bank Conflict", applied to 128-bit accesses).
//   B: BK rows x BN n, k-major as in global memory, row stride SB = BN + 8.
//      A lane reads one word; the two lane halves read rows 4 apart, and the
//      8-word pad places those two 32-word runs in different banks for a
//      64-bank LDS as well as a 32-bank one.
//
// Block -> tile mapping: gfx950 hands consecutive workgroups to its eight
// XCDs in turn, and each XCD has its own L2.  The block index is remapped so
// each XCD walks a contiguous run of tiles, and tiles are ordered in groups
// of GROUP_M tile rows so that the blocks resident on one XCD at a time
// share A row panels and B column panels in that XCD's L2.
#include "gemm_internal.h"

namespace gemmf32 {

namespace {
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_contiguous(int b, int nblocks) {
    const int per = nblocks / kXcds, extra = nblocks % kXcds;
    const int x = b % kXcds, local = b / kXcds;
    return x * per + min(x, extra) + local;
}
}  // namespace

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;     // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;               // 32x32 blocks per wave
    constexpr int SA = BK + 4, SB = BN + 8;
    constexpr int A_STAGE = BM * SA, B_STAGE = BK * SB;
    constexpr int A_CHUNKS = BM * BK / 4 / NT, B_CHUNKS = BK * BN / 4 / NT;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0, "tile shape");
    static_assert(A_CHUNKS * NT * 4 == BM * BK && B_CHUNKS * NT * 4 == BK * BN, "copy split");
    __shared__ __attribute__((aligned(16))) float lds[2 * (A_STAGE + B_STAGE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;

    // tile of this block
    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    floatx4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
            ra[u] = load4_ghost(p.A, m0 + r, p.M, k0 + c, p.K, p.lda);
        }
#pragma unroll
        for (int u = 0; u < B_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            rb[u] = load4_ghost(p.B, k0 + r, p.K, n0 + c, p.N, p.ldb);
        }
    };
    auto store_tiles = [&](int buf) {
        float* as = lds + buf * (A_STAGE + B_STAGE);
        float* bs = as + A_STAGE;
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
            *reinterpret_cast<floatx4*>(&as[r * SA + c]) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < B_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            *reinterpret_cast<floatx4*>(&bs[r * SB + c]) = rb[u];
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int phases = ceil_div(p.K, BK);
    if (phases > 0) {
        load_tiles(0);
        store_tiles(0);
    }
    __syncthreads();
    for (int ph = 0; ph < phases; ++ph) {
        const int cur = ph & 1;
        const bool more = ph + 1 < phases;
        if (more) load_tiles((ph + 1) * BK);
        const float* as = lds + cur * (A_STAGE + B_STAGE);
        const float* bs = as + A_STAGE;
#pragma unroll
        for (int kg = 0; kg < BK; kg += 8) {
            floatx4 a[FM];
            float b[FN][4];
#pragma unroll
            for (int f = 0; f < FM; ++f)
                a[f] = *reinterpret_cast<const floatx4*>(&as[(wm * WM + f * 32 + li) * SA + kg + 4 * lh]);
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    b[f][s] = bs[(kg + 4 * lh + s) * SB + wn * WN + f * 32 + li];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
        }
        if (more) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // Guarded store: register r of lane (li, lh) is row 8 (r/4) + 4 lh + r%4.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

namespace {
struct MfmaConfig {
    const char* name;
    int bm, bn, threads;
    hipError_t (*launch)(const GemmArgs&, hipStream_t, int, int, int, unsigned);
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                      unsigned blocks) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WAVES_M, WAVES_N>), dim3(blocks),
                       dim3(WAVES_M * WAVES_N * 64), 0, s, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

const MfmaConfig kConfigs[] = {
    {"mfma256x256_bk16_w2x2", 256, 256, 256, launch_cfg<256, 256, 16, 2, 2>},
    {"mfma128x128_bk16_w2x2", 128, 128, 256, launch_cfg<128, 128, 16, 2, 2>},
    {"mfma256x128_bk16_w2x2", 256, 128, 256, launch_cfg<256, 128, 16, 2, 2>},
    {"mfma128x128_bk32_w2x2", 128, 128, 256, launch_cfg<128, 128, 32, 2, 2>},
    {"mfma64x64_bk16_w2x2", 64, 64, 256, launch_cfg<64, 64, 16, 2, 2>},
};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
}  // namespace

int mfma_num_configs() { return kNumConfigs; }
const char* mfma_config_name(int c) { return (c >= 0 && c < kNumConfigs) ? kConfigs[c].name : nullptr; }

// Largest tile that still gives every CU at least one workgroup.
int mfma_pick_config(int M, int N, int /*K*/) {
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    if (t256 >= 256) return 0;
    if (t128 >= 256) return 1;
    return 4;
}

// Returns hipErrorInvalidValue when the grid would exceed the launch limits.
hipError_t launch_mfma(const GemmArgs& p, hipStream_t s, int config) {
    const MfmaConfig& c = kConfigs[(config >= 0 && config < kNumConfigs) ? config : 0];
    const int tiles_m = ceil_div(p.M, c.bm), tiles_n = ceil_div(p.N, c.bn);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks * c.threads > 0xFFFFFFFFll || blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const int group_m = 8;
    return c.launch(p, s, tiles_m, tiles_n, group_m, (unsigned)blocks);
}

}  // namespace gemmf32
