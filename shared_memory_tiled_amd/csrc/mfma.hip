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
//   A: BM rows x BK k, m-major as in global memory.  Register-staged
//      kernels pad each row by 4 words (row stride BK + 4): the 16 rows that
//      one 128-bit read touches per LDS cycle then start on 16 different
//      4-bank groups.  Direct-copy kernels cannot pad (one copy instruction
//      fills 1 KB contiguously), so they permute the 16-byte chunks of each
//      row by an XOR with the row index instead, to the same effect.
//   B: BK rows x BN n, k-major as in global memory, row stride BN + 8.  A
//      lane reads one word; the two lane halves read rows 4 apart, and the
//      8-word pad puts those two 32-word runs in different banks.
// The bank rule is the first page's ("Bank Conflict": n distinct words in
// one bank serialise), measured on gfx950 rather than assumed: 128-bit LDS
// reads are served 16 lanes at a time from 64 banks.  A swizzle laid out for
// 32 banks (kept as a diagnostic variant) shows 1.34e8 conflict cycles at
// 8192^3; the 64-bank one shows none.
//
// Copies: register-staged kernels load the next phase's tiles into VGPRs
// during the current phase's math and store them to the other LDS stage
// after it.  Direct-copy kernels (global_load_lds_dwordx4) write the other
// stage while the current one is read, with no register staging and no LDS
// store instructions; a phase that reaches past the matrix edge falls back
// to ghost-zero loads through registers into the same layout.
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

// One lane's 16 bytes from global memory straight into LDS: the wave's 64
// lanes fill 1 KB starting at `dst` (wave-uniform), lane l at byte 16 l.
__device__ __forceinline__ void copy16_global_to_lds(const float* src, float* dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ __forceinline__ int xcd_contiguous(int b, int nblocks) {
    const int per = nblocks / kXcds, extra = nblocks % kXcds;
    const int x = b % kXcds, local = b / kXcds;
    return x * per + min(x, extra) + local;
}
}  // namespace

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DIRECT, int SWZ_BANKS>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;     // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;               // 32x32 blocks per wave
    // A rows: padded by 4 words, or (DIRECT) unpadded with the 16-byte chunks
    // of a row permuted by an XOR of the row index, see a_chunk() below.
    constexpr int SA = DIRECT ? BK : BK + 4, SB = BN + 8;
    constexpr int CPR = BK / 4;                 // 16-byte chunks per A row
    // rows of the A tile that fit in one sweep of SWZ_BANKS 4-byte banks
    constexpr int ROWS_PER_BANK_CYCLE = SWZ_BANKS / BK;
    constexpr int A_STAGE = BM * SA, B_STAGE = BK * SB;
    constexpr int A_CHUNKS = BM * BK / 4 / NT, B_CHUNKS = BK * BN / 4 / NT;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0, "tile shape");
    static_assert(A_CHUNKS * NT * 4 == BM * BK && B_CHUNKS * NT * 4 == BK * BN, "copy split");
    static_assert(!DIRECT || (BN == 256 && (BK == 16 || BK == 32) && (BM * BK / 256) % NW == 0 &&
                              BK % NW == 0), "direct-to-LDS copy shape");
    __shared__ __attribute__((aligned(16))) float lds[2 * (A_STAGE + B_STAGE)];

    // Physical 16-byte chunk of logical chunk lc in A-tile row r.  With the
    // XOR, the eight rows a 128-bit access touches per LDS cycle (32 banks,
    // 8 lanes) read eight different bank groups, and the eight chunks a
    // 1 KB direct copy writes per cycle do too -- the swizzle of the first
    // page's "Bank Conflict" section, on 16-byte chunks instead of words.
    auto a_chunk = [](int r, int lc) {
        return DIRECT ? (lc ^ ((r / ROWS_PER_BANK_CYCLE) % CPR)) : lc;
    };

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

    // Per-thread element offsets of this thread's copy chunks (phase 0); a
    // phase adds k0 to the A offsets and k0 * ldb to the B offsets.  (Not
    // used by the direct-copy kernels.)
    int64_t a_off[A_CHUNKS], b_off[B_CHUNKS];
#pragma unroll
    for (int u = 0; u < (DIRECT ? 0 : A_CHUNKS); ++u) {
        const int q = tid + u * NT;
        a_off[u] = (int64_t)(m0 + q / (BK / 4)) * p.lda + (q % (BK / 4)) * 4;
    }
#pragma unroll
    for (int u = 0; u < (DIRECT ? 0 : B_CHUNKS); ++u) {
        const int q = tid + u * NT;
        b_off[u] = (int64_t)(q / (BN / 4)) * p.ldb + n0 + (q % (BN / 4)) * 4;
    }
    // Interior tiles skip the ghost checks: the test is uniform over the
    // block, so the branch below never diverges within a wave.
    const bool tile_inside = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    floatx4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load_tiles = [&](int k0) {
        if (!DIRECT && tile_inside && k0 + BK <= p.K) {
            const float* __restrict__ a = p.A + k0;
            const float* __restrict__ b = p.B + (int64_t)k0 * p.ldb;
#pragma unroll
            for (int u = 0; u < A_CHUNKS; ++u) __builtin_memcpy(&ra[u], a + a_off[u], 16);
#pragma unroll
            for (int u = 0; u < B_CHUNKS; ++u) __builtin_memcpy(&rb[u], b + b_off[u], 16);
            return;
        }
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
    // Direct copies global -> LDS (global_load_lds_dwordx4): each wave
    // instruction writes 1 KB of LDS contiguously, lane l at byte 16 l.  A:
    // instruction j of wave w fills rows R0 .. R0 + 64/CPR - 1 with
    // R0 = (w + j NW) 64/CPR; B: instruction j of wave w fills row w + j NW.
    constexpr int A_DIRECT = DIRECT ? BM * BK / 256 / NW : 0;
    constexpr int B_DIRECT = DIRECT ? BK / NW : 0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int64_t a_doff[A_DIRECT > 0 ? A_DIRECT : 1], b_doff[B_DIRECT > 0 ? B_DIRECT : 1];
    if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < A_DIRECT; ++j) {
            const int r = (wave_u + j * NW) * (64 / CPR) + lane / CPR;
            const int lc = a_chunk(r, lane % CPR);       // the XOR is its own inverse
            a_doff[j] = (int64_t)(m0 + r) * p.lda + 4 * lc;
        }
#pragma unroll
        for (int j = 0; j < B_DIRECT; ++j)
            b_doff[j] = (int64_t)(wave_u + j * NW) * p.ldb + n0 + 4 * lane;
    }
    auto direct_tiles = [&](int k0, int buf) {
        float* as = lds + buf * (A_STAGE + B_STAGE);
        float* bs = as + A_STAGE;
        const float* a = p.A + k0;
        const float* b = p.B + (int64_t)k0 * p.ldb;
#pragma unroll
        for (int j = 0; j < A_DIRECT; ++j)
            copy16_global_to_lds(a + a_doff[j], as + (wave_u + j * NW) * (64 / CPR) * SA);
#pragma unroll
        for (int j = 0; j < B_DIRECT; ++j)
            copy16_global_to_lds(b + b_doff[j], bs + (wave_u + j * NW) * SB);
    };

    // Ghost phases of the direct-copy kernels: load and store chunk by chunk
    // (no registers held across the math; these phases are rare).
    auto ghost_tiles_now = [&](int k0, int buf) {
        float* as = lds + buf * (A_STAGE + B_STAGE);
        float* bs = as + A_STAGE;
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
            *reinterpret_cast<floatx4*>(&as[r * SA + 4 * a_chunk(r, c / 4)]) =
                load4_ghost(p.A, m0 + r, p.M, k0 + c, p.K, p.lda);
        }
#pragma unroll
        for (int u = 0; u < B_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            *reinterpret_cast<floatx4*>(&bs[r * SB + c]) = load4_ghost(p.B, k0 + r, p.K, n0 + c, p.N, p.ldb);
        }
    };

    auto store_tiles = [&](int buf) {
        float* as = lds + buf * (A_STAGE + B_STAGE);
        float* bs = as + A_STAGE;
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = q / (BK / 4), c = (q % (BK / 4)) * 4;
            *reinterpret_cast<floatx4*>(&as[r * SA + 4 * a_chunk(r, c / 4)]) = ra[u];
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
    // A phase is copied directly into LDS when it lies wholly inside the
    // matrices; ghost phases go through registers (load4_ghost + LDS store).
    auto direct_ok = [&](int k0) { return DIRECT && tile_inside && k0 + BK <= p.K; };
    if (phases > 0) {
        if constexpr (DIRECT) {
            if (direct_ok(0)) direct_tiles(0, 0);
            else ghost_tiles_now(0, 0);
        } else {
            load_tiles(0);
            store_tiles(0);
        }
    }
    if constexpr (DIRECT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int ph = 0; ph < phases; ++ph) {
        const int cur = ph & 1;
        const bool more = ph + 1 < phases;
        if constexpr (DIRECT) {
            if (more) {
                if (direct_ok((ph + 1) * BK)) direct_tiles((ph + 1) * BK, cur ^ 1);
                else ghost_tiles_now((ph + 1) * BK, cur ^ 1);
            }
        } else if (more) {
            load_tiles((ph + 1) * BK);
        }
        const float* as = lds + cur * (A_STAGE + B_STAGE);
        const float* bs = as + A_STAGE;
#pragma unroll
        for (int kg = 0; kg < BK; kg += 8) {
            floatx4 a[FM];
            float b[FN][4];
#pragma unroll
            for (int f = 0; f < FM; ++f)
            {
                const int r = wm * WM + f * 32 + li;
                a[f] = *reinterpret_cast<const floatx4*>(&as[r * SA + 4 * a_chunk(r, kg / 4 + lh)]);
            }
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
        if (!DIRECT && more) store_tiles(cur ^ 1);
        // The direct copies write LDS behind the compiler's back: wait for
        // them, and tell the compiler that LDS changed across the barrier.
        if constexpr (DIRECT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if constexpr (DIRECT) asm volatile("" ::: "memory");
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

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DIRECT = false, int SWZ = 64>
hipError_t launch_cfg(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                      unsigned blocks) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WAVES_M, WAVES_N, DIRECT, SWZ>), dim3(blocks),
                       dim3(WAVES_M * WAVES_N * 64), 0, s, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

const MfmaConfig kConfigs[] = {
    // register-staged copies (global -> VGPR -> LDS), padded A rows
    {"mfma256x256_bk16_w2x2", 256, 256, 256, launch_cfg<256, 256, 16, 2, 2>},
    {"mfma128x128_bk16_w2x2", 128, 128, 256, launch_cfg<128, 128, 16, 2, 2>},
    {"mfma256x128_bk16_w2x2", 256, 128, 256, launch_cfg<256, 128, 16, 2, 2>},
    {"mfma128x128_bk32_w2x2", 128, 128, 256, launch_cfg<128, 128, 32, 2, 2>},
    {"mfma64x64_bk16_w2x2", 64, 64, 256, launch_cfg<64, 64, 16, 2, 2>},
    {"mfma256x256_bk32_w2x4", 256, 256, 512, launch_cfg<256, 256, 32, 2, 4>},
    {"mfma128x256_bk16_w2x2", 128, 256, 256, launch_cfg<128, 256, 16, 2, 2>},
    // direct copies (global -> LDS), XOR-swizzled A rows
    {"mfma256x256_bk32_w2x4_direct", 256, 256, 512, launch_cfg<256, 256, 32, 2, 4, true, 64>},
    {"mfma256x256_bk16_w2x4_direct", 256, 256, 512, launch_cfg<256, 256, 16, 2, 4, true, 64>},
    {"mfma256x256_bk32_w4x2_direct", 256, 256, 512, launch_cfg<256, 256, 32, 4, 2, true, 64>},
    // the same swizzle laid out for a 32-bank LDS: kept to show, in the bank
    // conflict counter, that gfx950 serves 128-bit reads from 64 banks
    {"mfma256x256_bk32_w2x4_direct_swz32", 256, 256, 512, launch_cfg<256, 256, 32, 2, 4, true, 32>},
};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
}  // namespace

int mfma_num_configs() { return kNumConfigs; }
const char* mfma_config_name(int c) { return (c >= 0 && c < kNumConfigs) ? kConfigs[c].name : nullptr; }

// Largest tile that still gives every CU at least one workgroup: 256 x 256
// with eight waves (two per SIMD, so one wave's barrier or LDS wait is
// covered by the other's matrix instructions) and direct global -> LDS
// copies once there are 256 such tiles.
int mfma_pick_config(int M, int N, int /*K*/) {
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    if (t256 >= 256) return 7;
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
