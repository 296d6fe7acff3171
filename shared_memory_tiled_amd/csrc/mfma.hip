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
// The same chapter runs the backward products X^T dY and dY W^T on the same
// tile kernel; here either factor may be stored transposed (op(A), op(B)).
//
// v_mfma_f32_32x32x2_f32: D(32x32) += A(32x2) B(2x32) per wave, 16 passes.
// Lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator
// register r of lane l holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// The order of the k terms inside a phase is free (the sum is the same up
// to rounding), so for each group of 8 k values lane half h = l / 32 feeds
// k = kg + 4h + s to the s-th of four instructions.  A lane's four operands
// of one factor are then four consecutive k values of one row of op(X).
// The k order depends only on the tile shape, never on how a factor is
// stored, so op(A) = A^T gives the same bits as A stored untransposed.
//
// Each factor is an MN x K matrix (MN = M for A, N for B) stored either
// k-contiguous (element (mn, k) at X[mn ld + k]: A as stored, B stored
// transposed) or mn-contiguous (X[k ld + mn]: B as stored, A stored
// transposed).  Its LDS tile keeps the stored orientation:
//   k-contiguous: MN rows of BK k values.  A lane's four k values are one
//      128-bit read.  Register-staged kernels pad rows by 4 words (row
//      stride BK + 4): the 16 rows one 128-bit read touches per LDS cycle
//      then start on 16 different 4-bank groups.  Direct-copy kernels cannot
//      pad (one copy instruction fills 1 KB contiguously), so they permute
//      the 16-byte chunks of each row by an XOR with the row index instead.
//   mn-contiguous: BK rows of MN values, row stride MN + 8.  A lane reads
//      its four k values as four words; the two lane halves read rows 4
//      apart, and the 8-word pad puts those two 32-word runs in different
//      banks.
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
// of group_m tile rows so that the blocks resident on one XCD at a time
// share A row panels and B column panels in that XCD's L2.
#include "launch.h"

#include <type_traits>

namespace gemmf32 {

namespace {

// One lane's 16 bytes from global memory straight into LDS: the wave's 64
// lanes fill 1 KB starting at `dst` (wave-uniform), lane l at byte 16 l.
__device__ __forceinline__ void copy16_global_to_lds(const float* src, float* dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Where one factor lives: stored matrix, leading dimension, extent along mn
// (M or N) and along k.
struct Factor {
    const float* X;
    int64_t ld;
    int mn_ext, k_ext;
};

// One factor's tile: MNT x BK values of op(X) per stage, copied by NT
// threads (NW waves).  KC: the factor is stored k-contiguous.  MC_PAD: the
// pad of an mn-contiguous row (8 words when two lane groups read rows 4
// apart, 4 words when four lane groups do: their 16-word runs then start 16
// banks apart).
template <int MNT, int BK, bool KC, bool DIRECT, int SWZ_BANKS, int NT, int NW, int MC_PAD = 8>
struct OperandTile {
    static constexpr int STRIDE = KC ? (DIRECT ? BK : BK + 4) : MNT + MC_PAD;
    static constexpr int WORDS = KC ? MNT * STRIDE : BK * STRIDE;    // per stage
    static constexpr int CPR = KC ? BK / 4 : MNT / 4;   // 16-byte chunks per stored row
    static constexpr int CHUNKS = MNT * BK / 4 / NT;    // copy chunks per thread
    static constexpr int ROWS_PER_SWEEP = SWZ_BANKS / BK;
    static constexpr int COPIES = !DIRECT ? 0 : (KC ? MNT * BK / 256 / NW : BK / NW);
    static_assert(CHUNKS * NT * 4 == MNT * BK, "copy split");
    static_assert(!DIRECT || (KC ? ((MNT * BK / 256) % NW == 0 && (BK == 16 || BK == 32))
                                 : (MNT == 256 && BK % NW == 0)),
                  "direct-copy tile shape");

    // Stored (row, col) of copy chunk q: rows are mn (KC) or k (MC).
    __device__ static int chunk_row(int q) { return q / CPR; }
    __device__ static int chunk_col(int q) { return (q % CPR) * 4; }
    // Physical position of 16-byte chunk lc in k-contiguous row r.
    __device__ static int phys(int r, int lc) {
        return (KC && DIRECT) ? (lc ^ ((r / ROWS_PER_SWEEP) % (BK / 4))) : lc;
    }
    // LDS word of the chunk that starts at stored (row, col), col % 4 == 0.
    __device__ static int word(int row, int col) {
        return KC ? row * STRIDE + 4 * phys(row, col / 4) : row * STRIDE + col;
    }
    // op(X)[mn0 + r][k0 + c .. c+3] as stored chunk, with ghost zeros.
    __device__ static floatx4 ghost_load(const Factor& f, int mn0, int k0, int row, int col) {
        return KC ? load4_ghost(f.X, mn0 + row, f.mn_ext, k0 + col, f.k_ext, f.ld)
                  : load4_ghost(f.X, k0 + row, f.k_ext, mn0 + col, f.mn_ext, f.ld);
    }
    // Element offset of stored (row, col) of the phase-0 tile; a phase adds
    // phase_step(k0).
    __device__ static int64_t offset(const Factor& f, int mn0, int row, int col) {
        return KC ? (int64_t)(mn0 + row) * f.ld + col : (int64_t)row * f.ld + mn0 + col;
    }
    __device__ static int64_t phase_step(const Factor& f, int k0) {
        return KC ? (int64_t)k0 : (int64_t)k0 * f.ld;
    }
    // Four k values (k = kg + 4h + s, s = 0..3) of row mn of op(X).
    __device__ static floatx4 fragment(const float* stage, int mn, int kg, int h) {
        if constexpr (KC) {
            return *reinterpret_cast<const floatx4*>(&stage[word(mn, kg + 4 * h)]);
        } else {
            floatx4 v;
#pragma unroll
            for (int s = 0; s < 4; ++s) v[s] = stage[(kg + 4 * h + s) * STRIDE + mn];
            return v;
        }
    }
    // Direct copy j of a wave: the stored rows it fills, and lane l's source.
    //   KC: rows R0 .. R0 + 64/CPR - 1 with R0 = (w + j NW) 64/CPR; lane l
    //       fills physical chunk l % CPR of row R0 + l / CPR.
    //   MC: row w + j NW; lane l fills columns 4l .. 4l + 3.
    __device__ static int copy_first_row(int wave, int j) {
        return KC ? (wave + j * NW) * (64 / CPR) : wave + j * NW;
    }
    __device__ static int64_t copy_offset(const Factor& f, int mn0, int wave, int j, int lane) {
        if constexpr (KC) {
            const int r = copy_first_row(wave, j) + lane / CPR;
            return (int64_t)(mn0 + r) * f.ld + 4 * phys(r, lane % CPR);   // XOR is its own inverse
        } else {
            return (int64_t)copy_first_row(wave, j) * f.ld + mn0 + 4 * lane;
        }
    }
};
}  // namespace

// MI: the matrix instruction, v_mfma_f32_32x32x2_f32 (32) or
// v_mfma_f32_16x16x4_f32 (16).  The 16x16 form does the same work per cycle
// with a quarter of the accumulator block per instruction: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16], and accumulator register r holds
// D[4 (l / 16) + r][l % 16].  For each group of 16 k values the lane group
// g = l / 16 feeds k = kg + 4g + s to the s-th of four instructions, so a
// lane again reads four consecutive k values of one row.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DIRECT, int SWZ_BANKS,
          bool TRANS_A, bool TRANS_B, int MI = 32>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;     // wave tile
    constexpr int FM = WM / MI, FN = WN / MI;               // MI x MI blocks per wave
    constexpr int KG = MI == 32 ? 8 : 16;                   // k values per group of four instructions
    constexpr int NACC = MI == 32 ? 16 : 4;                 // accumulator registers per block
    using Acc = std::conditional_t<MI == 32, floatx16, floatx4>;
    static_assert(MI == 32 || MI == 16, "matrix instruction");
    static_assert(WM % MI == 0 && WN % MI == 0 && BK % KG == 0, "tile shape");
    constexpr int MC_PAD = MI == 32 ? 8 : 4;
    using TA = OperandTile<BM, BK, !TRANS_A, DIRECT, SWZ_BANKS, NT, NW, MC_PAD>;
    using TB = OperandTile<BN, BK, TRANS_B, DIRECT, SWZ_BANKS, NT, NW, MC_PAD>;
    constexpr int STAGE = TA::WORDS + TB::WORDS;
    __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & (MI - 1), lh = lane / MI;       // row in block, lane group

    // tile of this block
    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    const Factor fa{p.A, p.lda, p.M, p.K};
    const Factor fb{p.B, p.ldb, p.N, p.K};
    // Interior tiles skip the ghost checks: the test is uniform over the
    // block, so the branches below never diverge within a wave.
    const bool tile_inside = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    // --- register-staged copies (not used by the direct-copy kernels) ---
    int64_t a_off[DIRECT ? 1 : TA::CHUNKS], b_off[DIRECT ? 1 : TB::CHUNKS];
    floatx4 ra[DIRECT ? 1 : TA::CHUNKS], rb[DIRECT ? 1 : TB::CHUNKS];
    if constexpr (!DIRECT) {
#pragma unroll
        for (int u = 0; u < TA::CHUNKS; ++u) {
            const int q = tid + u * NT;
            a_off[u] = TA::offset(fa, m0, TA::chunk_row(q), TA::chunk_col(q));
        }
#pragma unroll
        for (int u = 0; u < TB::CHUNKS; ++u) {
            const int q = tid + u * NT;
            b_off[u] = TB::offset(fb, n0, TB::chunk_row(q), TB::chunk_col(q));
        }
    }
    auto load_tiles = [&](int k0) {
        if constexpr (!DIRECT) {
            if (tile_inside && k0 + BK <= p.K) {
                const float* a = p.A + TA::phase_step(fa, k0);
                const float* b = p.B + TB::phase_step(fb, k0);
#pragma unroll
                for (int u = 0; u < TA::CHUNKS; ++u) __builtin_memcpy(&ra[u], a + a_off[u], 16);
#pragma unroll
                for (int u = 0; u < TB::CHUNKS; ++u) __builtin_memcpy(&rb[u], b + b_off[u], 16);
                return;
            }
#pragma unroll
            for (int u = 0; u < TA::CHUNKS; ++u) {
                const int q = tid + u * NT;
                ra[u] = TA::ghost_load(fa, m0, k0, TA::chunk_row(q), TA::chunk_col(q));
            }
#pragma unroll
            for (int u = 0; u < TB::CHUNKS; ++u) {
                const int q = tid + u * NT;
                rb[u] = TB::ghost_load(fb, n0, k0, TB::chunk_row(q), TB::chunk_col(q));
            }
        }
    };
    auto store_tiles = [&](int buf) {
        if constexpr (!DIRECT) {
            float* as = lds + buf * STAGE;
            float* bs = as + TA::WORDS;
#pragma unroll
            for (int u = 0; u < TA::CHUNKS; ++u) {
                const int q = tid + u * NT;
                *reinterpret_cast<floatx4*>(&as[TA::word(TA::chunk_row(q), TA::chunk_col(q))]) = ra[u];
            }
#pragma unroll
            for (int u = 0; u < TB::CHUNKS; ++u) {
                const int q = tid + u * NT;
                *reinterpret_cast<floatx4*>(&bs[TB::word(TB::chunk_row(q), TB::chunk_col(q))]) = rb[u];
            }
        }
    };

    // --- direct copies global -> LDS ---
    int64_t a_doff[TA::COPIES > 0 ? TA::COPIES : 1], b_doff[TB::COPIES > 0 ? TB::COPIES : 1];
    if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < TA::COPIES; ++j) a_doff[j] = TA::copy_offset(fa, m0, wave_u, j, lane);
#pragma unroll
        for (int j = 0; j < TB::COPIES; ++j) b_doff[j] = TB::copy_offset(fb, n0, wave_u, j, lane);
    }
    auto direct_tiles = [&](int k0, int buf) {
        float* as = lds + buf * STAGE;
        float* bs = as + TA::WORDS;
        const float* a = p.A + TA::phase_step(fa, k0);
        const float* b = p.B + TB::phase_step(fb, k0);
#pragma unroll
        for (int j = 0; j < TA::COPIES; ++j)
            copy16_global_to_lds(a + a_doff[j], as + TA::copy_first_row(wave_u, j) * TA::STRIDE);
#pragma unroll
        for (int j = 0; j < TB::COPIES; ++j)
            copy16_global_to_lds(b + b_doff[j], bs + TB::copy_first_row(wave_u, j) * TB::STRIDE);
    };
    // Ghost phases of the direct-copy kernels: load and store chunk by chunk
    // (no registers held across the math; these phases are rare).
    auto ghost_tiles_now = [&](int k0, int buf) {
        float* as = lds + buf * STAGE;
        float* bs = as + TA::WORDS;
#pragma unroll
        for (int u = 0; u < TA::CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = TA::chunk_row(q), c = TA::chunk_col(q);
            *reinterpret_cast<floatx4*>(&as[TA::word(r, c)]) = TA::ghost_load(fa, m0, k0, r, c);
        }
#pragma unroll
        for (int u = 0; u < TB::CHUNKS; ++u) {
            const int q = tid + u * NT;
            const int r = TB::chunk_row(q), c = TB::chunk_col(q);
            *reinterpret_cast<floatx4*>(&bs[TB::word(r, c)]) = TB::ghost_load(fb, n0, k0, r, c);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.0f;

    const int phases = ceil_div(p.K, BK);
    // A phase is copied directly into LDS when it lies wholly inside the
    // matrices; ghost phases go through registers (load4_ghost + LDS store).
    auto direct_ok = [&](int k0) { return tile_inside && k0 + BK <= p.K; };
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
        const float* as = lds + cur * STAGE;
        const float* bs = as + TA::WORDS;
#pragma unroll
        for (int kg = 0; kg < BK; kg += KG) {
            floatx4 a[FM], b[FN];
#pragma unroll
            for (int f = 0; f < FM; ++f) a[f] = TA::fragment(as, wm * WM + f * MI + li, kg, lh);
#pragma unroll
            for (int f = 0; f < FN; ++f) b[f] = TB::fragment(bs, wn * WN + f * MI + li, kg, lh);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        if constexpr (MI == 32)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
                    }
        }
        if (!DIRECT && more) store_tiles(cur ^ 1);
        // The direct copies write LDS behind the compiler's back: wait for
        // them, and tell the compiler that LDS changed across the barrier.
        if constexpr (DIRECT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if constexpr (DIRECT) asm volatile("" ::: "memory");
    }

    // Guarded store: register r of lane (li, lh) is row 8 (r/4) + 4 lh + r%4
    // of its 32x32 block, or row 4 lh + r of its 16x16 block.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * MI + li;
#pragma unroll
            for (int r = 0; r < NACC; ++r) {
                const int row = m0 + wm * WM + i * MI +
                                (MI == 32 ? 8 * (r >> 2) + 4 * lh + (r & 3) : 4 * lh + r);
                if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

// Small products: KS groups of four waves share one output tile and split its
// phases between them (round r: group g takes phase r KS + g), each group
// with its own double-buffered LDS stages and register-staged copies (as the
// kernel above with !DIRECT).  A problem with few tiles then still has KS
// waves per SIMD to hide each other's latencies.  At the end the groups'
// accumulators meet in LDS and group 0 adds them in group order, so the
// result is deterministic; its rounding differs from the one-group kernels
// (each group sums its own phases first), within the same bound.
template <int BM, int BN, int BK, int KS, bool TRANS_A, bool TRANS_B>
__global__ __launch_bounds__(256 * KS)
void gemm_mfma_splitk_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NWG = 4, NTG = NWG * 64;                  // waves and threads per group
    constexpr int WM = BM / 2, WN = BN / 2;                 // 2 x 2 waves per group
    constexpr int FM = WM / 32, FN = WN / 32;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0 && KS >= 2, "tile shape");
    using TA = OperandTile<BM, BK, !TRANS_A, false, 64, NTG, NWG>;
    using TB = OperandTile<BN, BK, TRANS_B, false, 64, NTG, NWG>;
    constexpr int STAGE = TA::WORDS + TB::WORDS;
    constexpr int GROUP_WORDS = 2 * STAGE;
    constexpr int RED_WORDS = (KS - 1) * BM * BN;           // partial tiles of groups 1 .. KS-1
    constexpr int LDS_WORDS = KS * GROUP_WORDS > RED_WORDS ? KS * GROUP_WORDS : RED_WORDS;
    __shared__ __attribute__((aligned(16))) float lds[LDS_WORDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kg = __builtin_amdgcn_readfirstlane(tid / NTG);     // group (wave-uniform)
    const int gtid = tid % NTG;
    const int gw = gtid >> 6;                                     // wave within the group
    const int wm = gw / 2, wn = gw % 2;
    const int li = lane & 31, lh = lane >> 5;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    const Factor fa{p.A, p.lda, p.M, p.K};
    const Factor fb{p.B, p.ldb, p.N, p.K};
    const bool tile_inside = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    float* glds = lds + kg * GROUP_WORDS;

    int64_t a_off[TA::CHUNKS], b_off[TB::CHUNKS];
#pragma unroll
    for (int u = 0; u < TA::CHUNKS; ++u) {
        const int q = gtid + u * NTG;
        a_off[u] = TA::offset(fa, m0, TA::chunk_row(q), TA::chunk_col(q));
    }
#pragma unroll
    for (int u = 0; u < TB::CHUNKS; ++u) {
        const int q = gtid + u * NTG;
        b_off[u] = TB::offset(fb, n0, TB::chunk_row(q), TB::chunk_col(q));
    }
    floatx4 ra[TA::CHUNKS], rb[TB::CHUNKS];
    auto load_tiles = [&](int k0) {
        if (tile_inside && k0 + BK <= p.K) {
            const float* a = p.A + TA::phase_step(fa, k0);
            const float* b = p.B + TB::phase_step(fb, k0);
#pragma unroll
            for (int u = 0; u < TA::CHUNKS; ++u) __builtin_memcpy(&ra[u], a + a_off[u], 16);
#pragma unroll
            for (int u = 0; u < TB::CHUNKS; ++u) __builtin_memcpy(&rb[u], b + b_off[u], 16);
            return;
        }
#pragma unroll
        for (int u = 0; u < TA::CHUNKS; ++u) {
            const int q = gtid + u * NTG;
            ra[u] = TA::ghost_load(fa, m0, k0, TA::chunk_row(q), TA::chunk_col(q));
        }
#pragma unroll
        for (int u = 0; u < TB::CHUNKS; ++u) {
            const int q = gtid + u * NTG;
            rb[u] = TB::ghost_load(fb, n0, k0, TB::chunk_row(q), TB::chunk_col(q));
        }
    };
    auto store_tiles = [&](int buf) {
        float* as = glds + buf * STAGE;
        float* bs = as + TA::WORDS;
#pragma unroll
        for (int u = 0; u < TA::CHUNKS; ++u) {
            const int q = gtid + u * NTG;
            *reinterpret_cast<floatx4*>(&as[TA::word(TA::chunk_row(q), TA::chunk_col(q))]) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < TB::CHUNKS; ++u) {
            const int q = gtid + u * NTG;
            *reinterpret_cast<floatx4*>(&bs[TB::word(TB::chunk_row(q), TB::chunk_col(q))]) = rb[u];
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
    const int rounds = ceil_div(phases, KS);
    // Every wave runs every round (one barrier each); a group whose phase of
    // the round lies past K only skips its copies and its math.
    if (kg < phases) {
        load_tiles(kg * BK);
        store_tiles(0);
    }
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        const int cur = r & 1;
        const int ph = r * KS + kg, ph_next = ph + KS;
        if (ph_next < phases) load_tiles(ph_next * BK);
        if (ph < phases) {
            const float* as = glds + cur * STAGE;
            const float* bs = as + TA::WORDS;
#pragma unroll
            for (int kk = 0; kk < BK; kk += 8) {
                floatx4 a[FM], b[FN];
#pragma unroll
                for (int f = 0; f < FM; ++f) a[f] = TA::fragment(as, wm * WM + f * 32 + li, kk, lh);
#pragma unroll
                for (int f = 0; f < FN; ++f) b[f] = TB::fragment(bs, wn * WN + f * 32 + li, kk, lh);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
            }
        }
        if (ph_next < phases) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // Groups 1 .. KS-1 leave their partial tiles in LDS (register r of lane l
    // of wave w at word ((g - 1) NWG + w) FM FN 16 64 + (i FN + j) 16 64 + 64 r
    // + l: consecutive lanes, consecutive words); group 0 adds them in order.
    constexpr int PER_WAVE = FM * FN * 16 * 64;
    if (kg > 0) {
        float* red = lds + ((kg - 1) * NWG + gw) * PER_WAVE;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[((i * FN + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll 1
        for (int gg = 1; gg < KS; ++gg) {
            const float* red = lds + ((gg - 1) * NWG + gw) * PER_WAVE;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * FN + j) * 16 + r) * 64 + lane];
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
}

namespace {
using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t, int, int, int, unsigned);

struct MfmaConfig {
    const char* name;
    int bm, bn, threads, group_m;
    LaunchFn launch[4];          // by 2 op_a + op_b; null: op pair not built for this config
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DIRECT, int SWZ, bool TRA, bool TRB,
          int MI = 32>
hipError_t launch_one(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                      unsigned blocks) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WAVES_M, WAVES_N, DIRECT, SWZ, TRA, TRB, MI>),
                       dim3(blocks), dim3(WAVES_M * WAVES_N * 64), 0, s, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int KS, bool TRA, bool TRB>
hipError_t launch_splitk(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                         unsigned blocks) {
    hipLaunchKernelGGL((gemm_mfma_splitk_kernel<BM, BN, BK, KS, TRA, TRB>), dim3(blocks), dim3(256 * KS), 0, s, p,
                       tiles_m, tiles_n, group_m);
    return hipGetLastError();
}
#define SPLITK_OPS(BM, BN, BK, KS)                                                             \
    {launch_splitk<BM, BN, BK, KS, false, false>, launch_splitk<BM, BN, BK, KS, false, true>, \
     launch_splitk<BM, BN, BK, KS, true, false>, launch_splitk<BM, BN, BK, KS, true, true>}

// The four-wave scheduled kernel where it takes the problem, else the
// eight-wave 256 x 256 direct-copy kernel.
template <bool TRA, bool TRB>
hipError_t launch_sched_or_direct(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                  unsigned blocks) {
    if (sched_f32_fits(p, TRA, TRB)) return launch_sched_f32(p, s, TRA, TRB, group_m, 256);
    return launch_one<256, 256, 32, 2, 4, true, 64, TRA, TRB>(p, s, tiles_m, tiles_n, 8, blocks);
}
#define SCHED_OPS                                                                      \
    {launch_sched_or_direct<false, false>, launch_sched_or_direct<false, true>,          \
     launch_sched_or_direct<true, false>, launch_sched_or_direct<true, true>}
// The same schedule on 128 x 128 tiles, else the register-staged 128 x 128
// kernel.
template <bool TRA, bool TRB>
hipError_t launch_sched128_or_staged(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                     unsigned blocks) {
    if (sched_f32_fits(p, TRA, TRB)) return launch_sched_f32(p, s, TRA, TRB, group_m, 128);
    return launch_one<128, 128, 16, 2, 2, false, 64, TRA, TRB>(p, s, tiles_m, tiles_n, 8, blocks);
}
#define SCHED128_OPS                                                                         \
    {launch_sched128_or_staged<false, false>, launch_sched128_or_staged<false, true>,          \
     launch_sched128_or_staged<true, false>, launch_sched128_or_staged<true, true>}

// Four waves splitting the phases of a 64 x 64 tile, else the split-phase
// kernel with four groups of four waves.
template <bool TRA, bool TRB>
hipError_t launch_ksplit_or_splitk(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                   unsigned blocks) {
    if (ksplit_f32_fits(p, TRA, TRB)) return launch_ksplit_f32(p, s, TRA, TRB, group_m);
    return launch_splitk<64, 64, 32, 4, TRA, TRB>(p, s, tiles_m, tiles_n, group_m, blocks);
}
// Four waves splitting the phases of one 96 x 96 tile where it takes the
// problem, else configuration 20.
template <bool TRA, bool TRB>
hipError_t launch_ksplit96_or_ksplit(const GemmArgs& p, hipStream_t s, int, int, int group_m, unsigned) {
    if (ksplit96_f32_fits(p, TRA, TRB)) return launch_ksplit96_f32(p, s, TRA, TRB, group_m);
    return launch_mfma(p, s, 20, TRA, TRB);
}
// 64 x 64 tiles of 2 x 2 waves, one 32 x 32 block each over the whole K,
// from NST LDS stages (gemm_f32_tile64_kernel), where they take the
// problem, else configuration 20.
template <int NST, bool TRA, bool TRB>
hipError_t launch_tile64_or_ksplit(const GemmArgs& p, hipStream_t s, int, int, int group_m, unsigned) {
    if (sched_f32_fits(p, TRA, TRB)) return launch_tile64_f32(p, s, TRA, TRB, group_m, NST);
    return launch_mfma(p, s, 20, TRA, TRB);
}
#define TILE64_OPS(NST)                                                                          \
    {launch_tile64_or_ksplit<NST, false, false>, launch_tile64_or_ksplit<NST, false, true>,          \
     launch_tile64_or_ksplit<NST, true, false>, launch_tile64_or_ksplit<NST, true, true>}
#define KSPLIT96_OPS                                                                          \
    {launch_ksplit96_or_ksplit<false, false>, launch_ksplit96_or_ksplit<false, true>,          \
     launch_ksplit96_or_ksplit<true, false>, launch_ksplit96_or_ksplit<true, true>}
#define KSPLIT_OPS                                                                       \
    {launch_ksplit_or_splitk<false, false>, launch_ksplit_or_splitk<false, true>,          \
     launch_ksplit_or_splitk<true, false>, launch_ksplit_or_splitk<true, true>}

// Small output tiles whose k groups are split over the waves of a block
// (small.hip).
template <int SHAPE, bool TRA, bool TRB>
hipError_t launch_small_cfg(const GemmArgs& p, hipStream_t s, int, int, int, unsigned) {
    return launch_small_f32(p, s, TRA, TRB, SHAPE);
}
#define SMALL_OPS(SHAPE)                                                                  \
    {launch_small_cfg<SHAPE, false, false>, launch_small_cfg<SHAPE, false, true>,          \
     launch_small_cfg<SHAPE, true, false>, launch_small_cfg<SHAPE, true, true>}

// NN only (diagnostic layouts) or all four op combinations.
#define NN_ONLY(BM, BN, BK, WM, WN, D, S) \
    {launch_one<BM, BN, BK, WM, WN, D, S, false, false>, nullptr, nullptr, nullptr}
#define ALL_OPS(BM, BN, BK, WM, WN, D, S)                    \
    {launch_one<BM, BN, BK, WM, WN, D, S, false, false>,     \
     launch_one<BM, BN, BK, WM, WN, D, S, false, true>,      \
     launch_one<BM, BN, BK, WM, WN, D, S, true, false>,      \
     launch_one<BM, BN, BK, WM, WN, D, S, true, true>}
#define ALL_OPS_MI16(BM, BN, BK, WM, WN, D, S)                   \
    {launch_one<BM, BN, BK, WM, WN, D, S, false, false, 16>,     \
     launch_one<BM, BN, BK, WM, WN, D, S, false, true, 16>,      \
     launch_one<BM, BN, BK, WM, WN, D, S, true, false, 16>,      \
     launch_one<BM, BN, BK, WM, WN, D, S, true, true, 16>}

const MfmaConfig kConfigs[] = {
    // register-staged copies (global -> VGPR -> LDS), padded k-contiguous rows
    {"mfma256x256_bk16_w2x2", 256, 256, 256, 8, NN_ONLY(256, 256, 16, 2, 2, false, 64)},
    {"mfma128x128_bk16_w2x2", 128, 128, 256, 8, ALL_OPS(128, 128, 16, 2, 2, false, 64)},
    {"mfma256x128_bk16_w2x2", 256, 128, 256, 8, NN_ONLY(256, 128, 16, 2, 2, false, 64)},
    {"mfma128x128_bk32_w2x2", 128, 128, 256, 8, NN_ONLY(128, 128, 32, 2, 2, false, 64)},
    {"mfma64x64_bk16_w2x2", 64, 64, 256, 8, ALL_OPS(64, 64, 16, 2, 2, false, 64)},
    {"mfma256x256_bk32_w2x4", 256, 256, 512, 8, NN_ONLY(256, 256, 32, 2, 4, false, 64)},
    {"mfma128x256_bk16_w2x2", 128, 256, 256, 8, NN_ONLY(128, 256, 16, 2, 2, false, 64)},
    // direct copies (global -> LDS), XOR-swizzled k-contiguous rows
    {"mfma256x256_bk32_w2x4_direct", 256, 256, 512, 8, ALL_OPS(256, 256, 32, 2, 4, true, 64)},
    {"mfma256x256_bk16_w2x4_direct", 256, 256, 512, 8, NN_ONLY(256, 256, 16, 2, 4, true, 64)},
    {"mfma256x256_bk32_w4x2_direct", 256, 256, 512, 8, NN_ONLY(256, 256, 32, 4, 2, true, 64)},
    // the same swizzle laid out for a 32-bank LDS: kept to show, in the bank
    // conflict counter, that gfx950 serves 128-bit reads from 64 banks
    {"mfma256x256_bk32_w2x4_direct_swz32", 256, 256, 512, 8, NN_ONLY(256, 256, 32, 2, 4, true, 32)},
    // the default with tile-row groups of 4 and 16 instead of 8 (L2 reuse)
    {"mfma256x256_bk32_w2x4_direct_g4", 256, 256, 512, 4, NN_ONLY(256, 256, 32, 2, 4, true, 64)},
    {"mfma256x256_bk32_w2x4_direct_g16", 256, 256, 512, 16, NN_ONLY(256, 256, 32, 2, 4, true, 64)},
    // small products: the phases of one tile split over groups of four waves
    {"mfma64x64_bk16_w2x2_k4", 64, 64, 1024, 8, SPLITK_OPS(64, 64, 16, 4)},
    {"mfma64x64_bk32_w2x2_k4", 64, 64, 1024, 8, SPLITK_OPS(64, 64, 32, 4)},
    // the 256 x 256 direct-copy tile on v_mfma_f32_16x16x4_f32
    {"mfma256x256_bk32_w2x4_direct_mi16", 256, 256, 512, 8, ALL_OPS_MI16(256, 256, 32, 2, 4, true, 64)},
    // four waves of 128 x 128, instruction order fixed by the kernel
    {"mfma256x256_bk32_w2x2_sched", 256, 256, 256, 8, SCHED_OPS},
    {"mfma256x256_bk32_w2x2_sched_g4", 256, 256, 256, 4, SCHED_OPS},
    {"mfma128x128_bk32_w2x2_sched", 128, 128, 256, 8, SCHED128_OPS},
    {"mfma128x128_bk32_w2x2_sched_g16", 128, 128, 256, 16, SCHED128_OPS},
    // four waves, each the whole 64 x 64 tile over every fourth phase
    {"mfma64x64_bk32_w1x1_k4_sched", 64, 64, 1024, 8, KSPLIT_OPS},
    // small products: 16 x 16 or 32 x 32 tiles, k groups split over the waves
    {"mfma16x16_w4_small", 16, 16, 256, 8, SMALL_OPS(0)},
    {"mfma32x32_w4_small", 32, 32, 256, 8, SMALL_OPS(1)},
    {"mfma16x16_w8_small", 16, 16, 512, 8, SMALL_OPS(2)},
    // four waves, each the whole 96 x 96 tile over every fourth 16-deep phase
    {"mfma96x96_bk16_w1x1_k4_sched", 96, 96, 1024, 8, KSPLIT96_OPS},
    // four waves of one 32 x 32 block each over the whole K (2 x 2 per
    // tile), three LDS stages (three blocks to a CU); then the same tiles
    // with four stages (copies three phases ahead, two blocks to a CU) and
    // with two (four blocks to a CU)
    {"mfma64x64_bk32_w2x2_sched", 64, 64, 256, 8, TILE64_OPS(3)},
    {"mfma64x64_bk32_w2x2_4stage", 64, 64, 256, 8, TILE64_OPS(4)},
    {"mfma64x64_bk32_w2x2_2stage", 64, 64, 256, 8, TILE64_OPS(2)},
};
#undef NN_ONLY
#undef ALL_OPS
#undef ALL_OPS_MI16
#undef SCHED_OPS
#undef SCHED128_OPS
#undef SPLITK_OPS
#undef KSPLIT_OPS
#undef KSPLIT96_OPS
#undef TILE64_OPS
#undef SMALL_OPS
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
}  // namespace

int mfma_num_configs() { return kNumConfigs; }
const char* mfma_config_name(int c) { return (c >= 0 && c < kNumConfigs) ? kConfigs[c].name : nullptr; }

// Tile choice.  Shapes the four-wave schedule takes (mfma_sched.hip: K, M
// and N multiples of 4): 256 x 256 tiles when there are at least
// 256 of them and their rounds of 256 workgroups (one per CU) run at least
// 95 % full, else its 128 x 128 tiles (two workgroups per CU) when there are
// at least 128, else the split-phase 64 x 64 tiles.  Other shapes: 256 x
// 256 tiles on eight waves (direct copies, ghost phases at the edges) when
// their rounds run at least 80 % full (75 % when 128 x 128 tiles would not
// fill theirs to 90 %), else register-staged 128 x 128 tiles when at least
// 256 of them fill their rounds to 90 %, else 64 x 64 tiles with the phases
// of each tile split over four groups of four waves (16 waves per workgroup
// to hide latency; 32-deep phases when there are at most 256 such tiles,
// 16-deep otherwise).
//
// Then, for K of at least 448 and K, M and N multiples of 4, the 64 x 64
// tiles whose four waves split the phases (mfma_sched.hip) replace that
// choice when a cost model gives them the shorter time.  The model charges
// each round of 256 tiles the tile's work at a kernel's measured fraction
// of the matrix-core peak plus a fixed cost per tile (first copies, final
// store): four-wave 256 x 256 0.985 and 11 us, 128 x 128 0.975 and 5.3 us,
// eight-wave 256 x 256 0.92 and 11 us, register-staged 128 x 128 0.85 and
// 5.3 us, 64 x 64 with split phases 0.914 and 3 us (fitted to 31 shapes
// from 512^3 to 8192^3; below K = 448 the model misjudges them against
// two co-resident 128 x 128 workgroups per CU, e.g. at 3000 x 3000 x 384:
// there they only replace the split-phase tiles, from K = 384, three
// phases per wave).  The 96 x 96 k-split tiles (mfma_ksplit96.hip) replace
// the choice in turn where the model gives them the shorter time, at 0.9925
// and 12 us (fitted to 1536^3 and 4608^3, the fixed cost raised from 10 us so
// that 3584^3, 5.6 rounds of them against 12.25 rounds of 64 x 64 k-split
// tiles, keeps the latter, 2-3 % faster there; within 4 % of the measured
// time at 2048^3, 2560^3, 3072^3, 5120^3, 6144^3 and 7168^3).  Then 64 x 64
// tiles of 2 x 2 one-block waves over the whole K (gemm_f32_tile64_kernel,
// three LDS stages) replace the choice, from K = 256, where the model gives
// them the shorter time at 0.85 and 4 us once per launch (three of their
// blocks share a CU; fitted to 22 shapes with K from 256 to 5120: 3000^2 x
// 384 115 TFLOP/s against 98 on 128 x 128 tiles, 2048 x 3072 x 512 122
// against 106 on the k-split tiles, 3072^2 x 768 132 against 120, 1000 x
// 2000 x 500 99 against 92, 3000 x 7000 x 1024 131 against 123; with one
// block per CU, 1000^3, they lose, 102 against 105: a barrier every phase
// of 16 instructions against none in the k-split waves).  Last, products of at most 1024 output tiles of 16 x 16
// take the small-tile kernels (16 x 16 tiles on 8 waves up to 512 such
// tiles, else 32 x 32 tiles on 4 waves).  Every picked configuration
// is built for all four op combinations.
namespace {
// Modelled time (ns) of a configuration: rounds x (tile work / efficiency
// + fixed cost); tile work at the per-CU peak of 2 x 64 x 64 x K flops per
// 64 x 64 tile at 614.5 GFLOP/s, 13.33 ns per k.
double model_ns(int config, int M, int N, int K) {
    int tile;
    double rel, eff, fixed;
    switch (config) {
        case 16: tile = 256; rel = 16; eff = 0.985; fixed = 11000; break;
        case 18: tile = 128; rel = 4; eff = 0.975; fixed = 5300; break;
        case 7: tile = 256; rel = 16; eff = 0.92; fixed = 11000; break;
        case 1: tile = 128; rel = 4; eff = 0.85; fixed = 5300; break;
        case 20: tile = 64; rel = 1; eff = 0.914; fixed = 3000; break;
        case 24: tile = 96; rel = 2.25; eff = 0.9925; fixed = 12000; break;
        case 25: tile = 64; rel = 1; eff = 0.85; fixed = 4000; break;
        default: return 1e300;                    // the split-phase 64 x 64 tiles: never kept over 20
    }
    const int64_t tiles = (int64_t)ceil_div(M, tile) * ceil_div(N, tile);
    const double rounds = (double)((tiles + 255) / 256);
    // Configuration 25's blocks (32 KB of LDS) share a CU four at a time, so
    // the start and end of one overlap the work of others: its fixed cost is
    // paid once per launch, not per round.
    if (config == 25) return rounds * rel * 13.33 * K / eff + fixed;
    return rounds * (rel * 13.33 * K / eff + fixed);
}
}  // namespace

int mfma_pick_config(int M, int N, int K) {
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    const int64_t t64 = (int64_t)ceil_div(M, 64) * ceil_div(N, 64);
    const int64_t slots256 = (t256 + 255) / 256 * 256, slots128 = (t128 + 255) / 256 * 256;
    const int small = t64 <= 256 ? 14 : 13;
    int pick;
    if (K % 4 == 0 && K > 0 && M % 4 == 0 && N % 4 == 0) {
        if (t256 >= 256 && t256 * 20 >= slots256 * 19) pick = 16;
        else pick = t128 >= 128 ? 18 : small;
    } else {
        const bool fill128 = t128 * 10 >= slots128 * 9;
        if (t256 >= 256 && (t256 * 10 >= slots256 * 8 || (t256 * 4 >= slots256 * 3 && !fill128))) pick = 7;
        else if (t128 >= 256 && fill128) pick = 1;
        else pick = small;
    }
    const bool split_fits = K % 4 == 0 && M % 4 == 0 && N % 4 == 0;
    if (split_fits && ((pick == small && K >= 384) || (K >= 448 && model_ns(20, M, N, K) < model_ns(pick, M, N, K))))
        pick = 20;
    if (split_fits && K >= 448 && model_ns(24, M, N, K) < model_ns(pick, M, N, K)) pick = 24;
    if (split_fits && K >= 256 && model_ns(25, M, N, K) < model_ns(pick, M, N, K) && model_ns(pick, M, N, K) < 1e300)
        pick = 25;
    // Few output elements: small tiles whose k groups are split over the
    // waves of a block (small.hip), any shape and K.  Measured kernel times
    // (256^3: 3.9 us against 8.7 for the split-phase tiles; 512^3: 9.2
    // against 11.8 for the k-split tiles; 256 x 256 x 1024: 6.9 against
    // 18.4) put the crossover near 1024 tiles of 16 x 16 (640^3, 1600 such
    // tiles: the k-split tiles lead, 16.2 against 17.8 us).
    const int64_t t16 = (int64_t)ceil_div(M, 16) * ceil_div(N, 16);
    if (t16 <= 512) pick = 23;                   // 16 x 16 tiles, 8 waves
    else if (t16 <= 1024) pick = 22;             // 32 x 32 tiles, 4 waves
    return pick;
}

int mfma_config_group_m(int config) {
    return kConfigs[(config >= 0 && config < kNumConfigs) ? config : 0].group_m;
}

// hipErrorInvalidValue: the grid would exceed the launch limits.
// hipErrorNotSupported: this configuration is not built for the op pair.
hipError_t launch_mfma(const GemmArgs& p, hipStream_t s, int config, int op_a, int op_b) {
    const MfmaConfig& c = kConfigs[(config >= 0 && config < kNumConfigs) ? config : 0];
    const LaunchFn fn = c.launch[2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)];
    if (fn == nullptr) return hipErrorNotSupported;
    const int tiles_m = ceil_div(p.M, c.bm), tiles_n = ceil_div(p.N, c.bn);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks * c.threads > 0xFFFFFFFFll || blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    return fn(p, s, tiles_m, tiles_n, c.group_m, (unsigned)blocks);
}

}  // namespace gemmf32
