// mfma16.hip -- the mixed-precision product: bfloat16 or binary16 inputs,
// binary32 accumulation and result, on gfx950's 16-bit matrix instructions.
//
// The one-volume PMPP notes ("PMPP 단권화", deep-learning chapter) run the
// fully connected layer as a matrix product on matrix units that take FP16 or
// BF16 inputs and accumulate in FP32 ("FC Layer = GEMM", "Mixed Precision").
// This is that product with the tiled structure of the fp32 kernels: per
// phase a block stages an A tile and a B tile in LDS, ghost zeros past the
// matrix edges, double-buffered stages and one barrier per phase, a guarded
// store of the binary32 accumulators.
//
// v_mfma_f32_32x32x16_{bf16,f16}: D(32x32) += A(32x16) B(16x32) per wave.
// Lane l supplies eight values of row l % 32 of A and eight of column l % 32
// of B, the same eight k for both factors; accumulator register r of lane l
// holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], as for the fp32
// instruction.  Which k a lane half holds is free as long as both factors
// agree, so in the s-th 16-deep step of a phase lane half h takes
// k = 16 s + 8 h + 0..7: each lane's operand of either factor is then eight
// consecutive k of one row, one 128-bit LDS read.
//
// LDS layouts.  k-contiguous tiles: one 128-byte row of BK = 64 values per
// output row (A) or column (B), the 16-byte chunk c of row r at chunk
// position c ^ f(r), f(r) = ((r >> 1) ^ (r >> 4)) & 7 (the first page's XOR
// swizzle, on 16-byte chunks); a fragment is one 128-bit read, 16 lanes per
// LDS cycle reading rows R .. R+15 at one chunk (a row pair spans the 64
// banks and f gives the eight row pairs eight different positions).
// mn-contiguous tiles (a factor copied as stored with n, or m, along its
// rows): 64 k rows of the tile's columns, chunk c of row r at c ^ 4 (r % 4),
// read transposed with ds_read_b64_tr_b16 (see read_tr16).
//
// Kernels.  gemm16_kernel: A (M x K, k-contiguous in memory) is copied as
// stored, straight from global memory into LDS in interior phases of the
// large tiles (global_load_lds_dwordx4, each wave instruction fills 1 KB),
// else with 128-bit loads through registers; B (K x N) is either copied as
// stored into an mn-contiguous tile (the direct-copy configurations) or
// transposed through registers into k-contiguous rows (each thread loads a
// block of 8 k rows x 8 or 4 n and writes 128-bit LDS rows of 8 k values; 8
// lanes per store cycle write rows 4l + j, which f spreads over eight
// positions).  gemm16_sched_kernel: 256 x 256 tiles (edge tiles run whole)
// on four waves with an explicit instruction order, the default for large
// problems.
// gemm16_op_kernel: either factor stored transposed.
//
// Vector loads need 4-byte alignment (gfx9 runs global memory in unaligned
// mode; a dword-aligned multi-dword load is legal): operands whose base is
// only 2-byte aligned, or whose leading dimension is odd, take the same
// kernels with element-wise 16-bit loads.
#include "mfma16_common.h"

#include <type_traits>
#include <utility>

namespace gemmf32 {

namespace {


constexpr int kBK = 64;          // k values per phase = one 128-byte LDS row
constexpr int kCPR = kBK / 8;    // 16-byte chunks per LDS row

__host__ __device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 4)) & 7; }
// Element offset, inside a tile stage, of logical chunk c of row r.
__device__ __forceinline__ int lds_elem(int r, int c) { return r * kBK + 8 * (c ^ swz(r)); }

// One lane's 16 bytes from global memory straight into LDS: the wave's 64
// lanes fill 1 KB starting at `dst` (wave-uniform), lane l at byte 16 l.
__device__ __forceinline__ void copy16_to_lds(const uint16_t* src, uint16_t* dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int FMT>
__device__ __forceinline__ floatx16 mfma16(u32x4 a, u32x4 b, floatx16 c) {
    if constexpr (FMT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// Eight consecutive elements of row r from column c of a rows x cols matrix
// (leading dimension ld); slots outside the matrix are +0 and never loaded.
template <bool VEC>
__device__ __forceinline__ u32x4 load8_ghost(const uint16_t* __restrict__ base, int r, int rows, int c,
                                             int cols, int64_t ld) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows) {
        const uint16_t* q = base + (int64_t)r * ld + c;
        if (VEC && c + 8 <= cols) {
            __builtin_memcpy(&v, q, 16);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c + e < cols) v[e >> 1] |= (unsigned)q[e] << (16 * (e & 1));
        }
    }
    return v;
}

// Four consecutive elements of row r from column c, ghost zeros as above.
template <bool VEC>
__device__ __forceinline__ u32x2 load4_ghost16(const uint16_t* __restrict__ base, int r, int rows, int c,
                                               int cols, int64_t ld) {
    u32x2 v = {0u, 0u};
    if (r < rows) {
        const uint16_t* q = base + (int64_t)r * ld + c;
        if (VEC && c + 4 <= cols) {
            __builtin_memcpy(&v, q, 8);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c + e < cols) v[e >> 1] |= (unsigned)q[e] << (16 * (e & 1));
        }
    }
    return v;
}

// Column j of an 8 x W block (W = 4 or 8) held as eight rows of W 16-bit
// values (u32x2 or u32x4 each), as one 128-bit row of eight values (row i in
// element i).
template <typename Row>
__device__ __forceinline__ u32x4 block_column(const Row (&v)[8], int j) {
    u32x4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const unsigned lo = v[2 * q][j >> 1], hi = v[2 * q + 1][j >> 1];
        t[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    return t;
}
}  // namespace

// BTR: B is copied into LDS as stored (k rows of n values, straight from
// global memory like A) and its fragments are read with ds_read_b64_tr_b16.
// The 16-byte chunk c of B row r sits at chunk position c ^ 4 (r % 4): the
// 32 lanes of one transposed read cover rows kb .. kb+3 and 32 consecutive n
// (four chunks), 16 distinct chunk positions, all 64 banks once.
template <int FMT, int BM, int BN, int WAVES_M, int WAVES_N, bool DIRECT, bool VEC, bool BTR>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm16_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;             // 32 x 32 blocks per wave
    constexpr int A_CHUNKS = BM * kCPR / NT;              // register-staged A chunks per thread
    // B is moved in blocks of 8 k rows x BW n: BW = 8 (128-bit loads) when the
    // blocks divide evenly among the threads, else BW = 4 (64-bit loads)
    constexpr int BW = ((kBK / 8) * (BN / 8)) % NT == 0 ? 8 : 4;
    constexpr int NBW = BN / BW;                          // n blocks per k-block row of B
    constexpr int B_BLOCKS = (kBK / 8) * NBW / NT;        // 8 x BW blocks of B per thread
    constexpr int A_COPIES = BM / 8 / NW;                 // direct 1 KB copies per wave
    constexpr int CPRB = BN / 8;                          // BTR: 16-byte chunks per B row
    constexpr int B_COPIES = kBK * BN * 2 / 1024 / NW;    // BTR: direct 1 KB copies per wave
    static_assert(!BTR || (DIRECT && CPRB >= 16 && 64 % CPRB == 0 && B_COPIES * NW * 1024 == kBK * BN * 2),
                  "transposed-read B tile");
    constexpr int STAGE = (BM + BN) * kBK;                // 16-bit elements per stage
    static_assert(WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(A_CHUNKS * NT == BM * kCPR && B_BLOCKS * NT == (kBK / 8) * NBW, "copy split");
    static_assert(!DIRECT || (VEC && A_COPIES * NW * 8 == BM), "direct copy split");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;

    // tile of this block: XCD-contiguous runs, in groups of group_m tile rows
    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;
    // Interior tiles with vector-aligned operands run their full phases on
    // straight-line loads (no ghost checks); edge tiles and a ragged last
    // phase take the ghost-zero loads.  The test is uniform over the block.
    const bool fast_tile = VEC && (m0 + BM <= p.M) && (n0 + BN <= p.N);

    // ---- A through registers (every phase when !DIRECT; ghost phases otherwise)
    u32x4 ra[A_CHUNKS];
    auto load_a_fast = [&](int k0) {
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT, r = q / kCPR, c = q % kCPR;
            __builtin_memcpy(&ra[u], p.A + (int64_t)(m0 + r) * p.lda + k0 + 8 * c, 16);
        }
    };
    auto load_a_ghost = [&](int k0) {
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT, r = q / kCPR, c = q % kCPR;
            ra[u] = load8_ghost<VEC>(p.A, m0 + r, p.M, k0 + 8 * c, p.K, p.lda);
        }
    };
    auto store_a = [&](int buf) {
        uint16_t* as = lds + buf * STAGE;
#pragma unroll
        for (int u = 0; u < A_CHUNKS; ++u) {
            const int q = tid + u * NT;
            *reinterpret_cast<u32x4*>(&as[lds_elem(q / kCPR, q % kCPR)]) = ra[u];
        }
    };
    // Direct copy j of this wave fills LDS rows R .. R+7, R = 8 (wave + j NW);
    // lane l writes physical chunk l % 8 of row R + l / 8, so it reads the
    // logical chunk (l % 8) ^ f(row) of global row m0 + row.
    int64_t a_doff[DIRECT ? A_COPIES : 1];
    if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < A_COPIES; ++j) {
            const int row = 8 * (wave_u + j * NW) + lane / 8;
            a_doff[j] = (int64_t)(m0 + row) * p.lda + 8 * ((lane % 8) ^ swz(row));
        }
    }
    auto direct_a = [&](int k0, int buf) {
        if constexpr (DIRECT) {
            uint16_t* as = lds + buf * STAGE;
            const uint16_t* a = p.A + k0;
#pragma unroll
            for (int j = 0; j < A_COPIES; ++j)
                copy16_to_lds(a + a_doff[j], as + 8 * (wave_u + j * NW) * kBK);
        }
    };

    // ---- B: 8 x BW blocks, q = tid + u NT: n block q % NBW, k block q / NBW
    using BRow = typename std::conditional<BW == 8, u32x4, u32x2>::type;
    BRow rb[BTR ? 1 : B_BLOCKS][8];
    auto load_b_fast = [&](int k0) {
#pragma unroll
        for (int u = 0; u < B_BLOCKS; ++u) {
            const int q = tid + u * NT, nb = q % NBW, kb = q / NBW;
            const uint16_t* b = p.B + (int64_t)(k0 + 8 * kb) * p.ldb + n0 + BW * nb;
#pragma unroll
            for (int i = 0; i < 8; ++i) __builtin_memcpy(&rb[u][i], b + i * p.ldb, 2 * BW);
        }
    };
    auto load_b_ghost = [&](int k0) {
#pragma unroll
        for (int u = 0; u < B_BLOCKS; ++u) {
            const int q = tid + u * NT, nb = q % NBW, kb = q / NBW;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (BW == 8)
                    rb[u][i] = load8_ghost<VEC>(p.B, k0 + 8 * kb + i, p.K, n0 + 8 * nb, p.N, p.ldb);
                else
                    rb[u][i] = load4_ghost16<VEC>(p.B, k0 + 8 * kb + i, p.K, n0 + 4 * nb, p.N, p.ldb);
            }
        }
    };
    // Row n = BW nb + j of the LDS tile gets column j of the block.  With
    // BW = 8 the eight lanes of one store cycle write rows 8 l + j, with
    // BW = 4 rows 4 l + j: f spreads both over eight chunk positions.
    auto store_b = [&](int buf) {
        uint16_t* bs = lds + buf * STAGE + BM * kBK;
#pragma unroll
        for (int u = 0; u < B_BLOCKS; ++u) {
            const int q = tid + u * NT, nb = q % NBW, kb = q / NBW;
#pragma unroll
            for (int j = 0; j < BW; ++j)
                *reinterpret_cast<u32x4*>(&bs[lds_elem(BW * nb + j, kb)]) = block_column(rb[u], j);
        }
    };

    // ---- BTR: B as stored.  Element offset of chunk c of B row r:
    auto b_elem = [](int r, int c) { return r * BN + 8 * (c ^ (4 * (r & 3))); };
    // Direct copy j of this wave fills B rows R .. R + 64/CPRB - 1 with
    // R = (64/CPRB) (wave + j NW); lane l writes physical chunk l % CPRB of
    // row R + l / CPRB.
    int64_t b_doff[BTR ? B_COPIES : 1];
    if constexpr (BTR) {
#pragma unroll
        for (int j = 0; j < B_COPIES; ++j) {
            const int row = (64 / CPRB) * (wave_u + j * NW) + lane / CPRB;
            b_doff[j] = (int64_t)row * p.ldb + n0 + 8 * ((lane % CPRB) ^ (4 * (row & 3)));
        }
    }
    auto direct_b = [&](int k0, int buf) {
        if constexpr (BTR) {
            uint16_t* bs = lds + buf * STAGE + BM * kBK;
            const uint16_t* b = p.B + (int64_t)k0 * p.ldb;
#pragma unroll
            for (int j = 0; j < B_COPIES; ++j)
                copy16_to_lds(b + b_doff[j], bs + (64 / CPRB) * (wave_u + j * NW) * BN);
        }
    };
    // Ghost phases of a BTR kernel: B rows loaded and stored chunk by chunk
    // (no registers held across the math; these phases are rare).
    auto ghost_b_now = [&](int k0, int buf) {
        if constexpr (BTR) {
            uint16_t* bs = lds + buf * STAGE + BM * kBK;
#pragma unroll
            for (int u = 0; u < kBK * CPRB / NT; ++u) {
                const int q = tid + u * NT, r = q / CPRB, c = q % CPRB;
                *reinterpret_cast<u32x4*>(&bs[b_elem(r, c)]) =
                    load8_ghost<VEC>(p.B, k0 + r, p.K, n0 + 8 * c, p.N, p.ldb);
            }
        }
    };
    // Transposed fragment of B: lane (g = lane / 16, j = lane % 16) addresses
    // row 16 s + 8 (g / 2) + 4 r + j / 4, column n + 16 (g % 2) + 4 (j % 4)
    // for reads r = 0, 1 (k 0..3 and 4..7 of its lane half).
    const int tr_g = lane >> 4, tr_j = lane & 15;
    auto read_b_tr = [&](const uint16_t* bs, int s, int f) {
        const int n = wn * WN + f * 32 + 16 * (tr_g & 1) + 4 * (tr_j & 3);
        u32x4 out;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 16 * s + 8 * (tr_g >> 1) + 4 * r + (tr_j >> 2);
            const u32x2 v = read_tr16(lds_addr(bs + b_elem(row, n >> 3) + 4 * ((n >> 2) & 1)));
            out[2 * r] = v[0];
            out[2 * r + 1] = v[1];
        }
        return out;
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // The fragments of 16-deep step s are read while the matrix instructions
    // of step s - 1 run (two register sets), so LDS latency hides behind them.
    auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int s, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
            a[f] = *reinterpret_cast<const u32x4*>(&as[lds_elem(wm * WM + f * 32 + li, 2 * s + lh)]);
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            if constexpr (BTR) b[f] = read_b_tr(bs, s, f);
            else b[f] = *reinterpret_cast<const u32x4*>(&bs[lds_elem(wn * WN + f * 32 + li, 2 * s + lh)]);
        }
    };
    // One wave per SIMD (128 x 128 wave tiles, accumulators in AGPRs): the
    // next step's fragment reads and the next stage's B stores are placed
    // among the matrix instructions explicitly.
    constexpr bool PIPE = FM * FN >= 16;
    // before_last() runs just before the last step's matrix instructions
    // (the next stage's stores: they write the other LDS stage).
    auto math = [&](int buf, auto&& before_last) {
        const uint16_t* as = lds + buf * STAGE;
        const uint16_t* bs = as + BM * kBK;
        u32x4 a[2][FM], b[2][FN];
        read_frags(as, bs, 0, a[0], b[0]);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            // this step's transposed reads were issued one step ago
            if constexpr (BTR) wait_tied(b[s & 1]);
            if (s + 1 < kBK / 16) {
                read_frags(as, bs, s + 1, a[(s + 1) & 1], b[(s + 1) & 1]);
                // keep the reads ahead of this step's matrix instructions
                if constexpr (PIPE) __builtin_amdgcn_sched_barrier(0);
            } else {
                before_last();
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<FMT>(a[s & 1][i], b[s & 1][j], acc[i][j]);
        }
        if constexpr (PIPE && !BTR) {
            // last step: one LDS store after each of the first matrix
            // instructions, the transposes in between
#pragma unroll
            for (int t = 0; t < B_BLOCKS * BW; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
        }
    };
    // The direct copies write LDS behind the compiler's back: wait for them,
    // and tell the compiler that LDS changed across the barrier.
    auto end_phase = [&]() {
        if constexpr (DIRECT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if constexpr (DIRECT) asm volatile("" ::: "memory");
    };
    // Tiles of the phase starting at k0 into stage buf, FAST (interior, full
    // phase) or with ghost zeros, issued now and stored by finish_tiles.
    auto start_tiles = [&](int k0, int buf, auto fast) {
        if constexpr (decltype(fast)::value) {
            if constexpr (DIRECT) direct_a(k0, buf);
            else load_a_fast(k0);
            if constexpr (BTR) direct_b(k0, buf);
            else load_b_fast(k0);
        } else {
            load_a_ghost(k0);
            if constexpr (BTR) ghost_b_now(k0, buf);
            else load_b_ghost(k0);
        }
    };
    auto finish_tiles = [&](int buf, auto fast) {
        if constexpr (!(DIRECT && decltype(fast)::value)) store_a(buf);
        if constexpr (!BTR) store_b(buf);
    };
    // One phase on stage ph & 1 while the next phase's tiles (PF: 0 none,
    // 1 fast, 2 ghost) go to the other stage.
    auto phase = [&](int ph, auto pf) {
        constexpr int PF = decltype(pf)::value;
        const int cur = ph & 1, k_next = (ph + 1) * kBK;
        if constexpr (PF == 1) start_tiles(k_next, cur ^ 1, std::true_type{});
        if constexpr (PF == 2) start_tiles(k_next, cur ^ 1, std::false_type{});
        // keep the next phase's loads ahead of the math, so their latency
        // hides behind it (the scheduler would otherwise sink them to their use)
        if constexpr (PF != 0) __builtin_amdgcn_sched_barrier(0);
        if constexpr (PIPE && PF == 1) {
            // the stores of the next stage go in among the last step's
            // matrix instructions
            math(cur, [&]() { finish_tiles(cur ^ 1, std::true_type{}); });
        } else {
            math(cur, []() {});
            // keep the loads' use (B's transpose, the LDS stores) after the math
            if constexpr (PF != 0) __builtin_amdgcn_sched_barrier(0);
            if constexpr (PF == 1) finish_tiles(cur ^ 1, std::true_type{});
            if constexpr (PF == 2) finish_tiles(cur ^ 1, std::false_type{});
        }
        end_phase();
    };
    using none = std::integral_constant<int, 0>;
    using fast = std::integral_constant<int, 1>;
    using ghost = std::integral_constant<int, 2>;

    const int phases = ceil_div(p.K, kBK);
    const int full = fast_tile ? p.K / kBK : 0;      // phases loaded straight (no ghosts)
    if (phases > 0) {
        if (full > 0) {
            start_tiles(0, 0, std::true_type{});
            finish_tiles(0, std::true_type{});
        } else {
            start_tiles(0, 0, std::false_type{});
            finish_tiles(0, std::false_type{});
        }
    }
    end_phase();
    int ph = 0;
    for (; ph + 1 < full; ++ph) phase(ph, fast{});          // next phase full: the hot loop
    for (; ph + 1 < phases; ++ph) phase(ph, ghost{});       // next phase ragged or edge tile
    if (ph < phases) phase(ph, none{});

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

// ---------------------------------------------------------------------------
// The scheduled kernel: 256 x 256 tiles of full phases (M and N multiples of
// 256, K of 64, vector-aligned operands under 2^31 bytes each), four waves of
// 128 x 128, one per SIMD, with every instruction of the K loop placed in
// program order.  Same LDS layouts as the kernels above except for the
// k-contiguous swizzle (below), and the same k order (so the same bits), but:
//  * Each step issues its 16 matrix instructions one at a time, with the next
//    step's fragment reads (two after each of the first ones) and the copies
//    of the next phase (one after each odd one) between them, so the reads'
//    latency and the copies' issue hide behind matrix work.  Scheduling
//    barriers keep the compiler from regrouping them.
//  * The last step's matrix instructions of each phase run after the
//    barrier, on fragments read before it, while the next phase's first
//    fragments are read: the SIMD has matrix work across the barrier.
//  * The copies of phase ph + 1 are issued between the barriers that end
//    phases ph - 1 and ph (eight with the deferred step, eight with step 0),
//    a whole phase ahead of their use.  They are buffer loads into LDS: base
//    and extent in a resource, the per-lane offset in a register, the phase's
//    k in the scalar offset, so they cost no vector instruction.
//  * Fragment read addresses are a per-lane base plus a compile-time offset
//    (step, fragment), and the bases move to the other stage once per phase:
//    besides the matrix instructions the loop holds only those 8 vector adds
//    per phase.  A vector ALU instruction between two matrix instructions
//    costs the matrix core about 14 cycles (measured on the fp32 kernel),
//    a lot against a 32-cycle instruction; scalar ones cost nothing.
// With two waves per SIMD (the kernels above) the waves of a SIMD drift
// apart within a phase and the younger one runs alone, its latencies
// exposed, while the older one waits at the barrier.
//
// Each factor's tile is one of two kinds (see gemm16_op_kernel):
//   KC (k-contiguous: A as stored, B stored transposed): 256 rows of 64 k,
//      chunk c of row r at c ^ ((r / 2) mod 8) (the 16 rows one read cycle
//      touches -- four 4-lane quads of a half-wave -- on 16 different 4-bank
//      groups; for
//      the rows 32 f + l % 32 a lane reads, the permutation depends on l
//      only, so fragment f is a compile-time offset); a fragment is one
//      128-bit read; a copy fills 8 rows;
//   MC (mn-contiguous: B as stored, A stored transposed): 64 k rows of 256
//      values, chunk c of row r at c ^ 4 (r % 4); a fragment is two
//      ds_read_b64_tr_b16 reads; a copy fills 2 rows.
// Both are 32 KB per stage: LDS holds A's stages at bytes 0 and 32768, B's at
// 65536 and 98304.
__host__ __device__ __forceinline__ constexpr int sched_swz(int r) { return (r >> 1) & 7; }

template <bool KC>
struct SchedTile {
    static constexpr int MNT = 256, NW = 4;
    static constexpr int READS = KC ? 4 : 8;      // LDS reads per step for 4 fragments
    // Copy j (0..7) of wave w: element offset, inside the tile stage, of the
    // first LDS element it fills, and lane l's stored (row, 8-value chunk).
    __host__ __device__ static int copy_dst(int w, int j) {
        return KC ? 8 * (w + j * NW) * kBK : 2 * (w + j * NW) * MNT;
    }
    // Byte offset of lane l's 16 bytes of copy j from the stored matrix's base
    // at k = 0 (mn0: the tile's first row or column of op(X)).
    __host__ __device__ static uint32_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        if constexpr (KC) {
            const int row = 8 * (w + j * NW) + lane / 8;
            return 2u * (uint32_t)((mn0 + row) * ld + 8 * ((lane % 8) ^ sched_swz(row)));
        } else {
            const int row = 2 * (w + j * NW) + lane / 32;
            return 2u * (uint32_t)(row * ld + mn0 + 8 * ((lane % 32) ^ (4 * (row & 3))));
        }
    }
    // k of lane l's 16 bytes of copy j of wave w, relative to the phase's
    // first k (KC: the first of its 8 values).
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        if constexpr (KC) {
            const int row = 8 * (w + j * NW) + lane / 8;
            return 8 * ((lane % 8) ^ sched_swz(row));
        } else {
            return 2 * (w + j * NW) + lane / 32;
        }
    }
    // Byte offset of the phase at k0 from the phase at 0.
    __host__ __device__ static int phase_bytes(int k0, int64_t ld) { return KC ? 2 * k0 : 2 * k0 * (int)ld; }
};

template <int FMT, bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm16_sched_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    constexpr int BM = 256, BN = 256, NW = 4, WM = 128, WN = 128, FM = 4, FN = 4;
    using TA = SchedTile<KCA>;
    using TB = SchedTile<KCB>;
    constexpr int TILE = 256 * kBK;                       // elements per tile stage
    constexpr int A_COPIES = 8, NCOPY = 16;               // 1 KB copies per wave and phase
    constexpr int NREAD = TA::READS + TB::READS;          // LDS reads per step
    static_assert(TILE * 2 == 32768 && NREAD <= 16, "stage layout");
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave_u / 2, wn = wave_u % 2;
    const int li = lane & 31, lh = lane >> 5;
    const int tr_g = lane >> 4, tr_j = lane & 15;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    // Copies 0..7 fill A's tile, 8..15 B's (byte offsets: the launcher keeps
    // both operands below 2^31 bytes).
    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        doff[j] = TA::copy_src(wave_u, j, lane, m0, p.lda);
        doff[A_COPIES + j] = TB::copy_src(wave_u, j, lane, n0, p.ldb);
    }
    constexpr int kRawBufferWord3 = 0x00020000;
    // Each descriptor ends exactly at its stored matrix's last element, and
    // a copy that must bring zeros gets them from a per-lane offset that by
    // itself lies at or past that end (the scalar offset, which holds the
    // phase, never decides it).  An edge tile's copies past the last row of
    // a k-contiguous factor have such offsets in every phase.  Past the last
    // column of an mn-contiguous factor they read the next row, which only
    // ever meets C entries outside the matrix, never stored.  The last
    // phase's copies take their own per-lane offsets (dlast) with the phase
    // folded in and a scalar offset of 0: K is a multiple of 8, its 16-byte
    // chunks or rows at k >= K are pointed past the end (kPastEnd), so they
    // copy zeros, and a chunk of the last row past the last column lies past
    // the end by its own offset.  A 16-byte chunk across the end of an
    // mn-contiguous factor's last row reads its dwords up to the
    // descriptor's end and zeros past it (the range check is per dword;
    // checked on MI355X); the factor's width is even, so no dword straddles
    // that end.  The 8-wave kernel's ghost phase has the same zeros, so both
    // still give the same bits.
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.A), (short)0, (int)(2 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.B), (short)0, (int)(2 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    const int P = ceil_div(p.K, kBK);
    constexpr uint32_t kPastEnd = 0x80000000u;              // beyond any descriptor here
    const int klast = (P - 1) * kBK;                        // the last phase's first k
    uint32_t dlast[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        const int ka = klast + TA::copy_k(wave_u, j, lane);
        const int kb = klast + TB::copy_k(wave_u, j, lane);
        dlast[j] = ka >= p.K ? kPastEnd : doff[j] + (uint32_t)TA::phase_bytes(klast, p.lda);
        dlast[A_COPIES + j] = kb >= p.K ? kPastEnd : doff[A_COPIES + j] + (uint32_t)TB::phase_bytes(klast, p.ldb);
    }
    // Copy j of the phase at k0 into stage buf; LAST: the phase is the last
    // (its offsets hold the phase; k0 is not used).
    auto copy = [&](int j, int k0, int buf, auto lastc) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(lastc)::value;
        const uint32_t voff = LAST ? dlast[j] : doff[j];
        if (j < A_COPIES) {
            const int soff = LAST ? 0 : TA::phase_bytes(k0, p.lda);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(lds + buf * TILE + TA::copy_dst(wave_u, j)), 16,
                (int)voff, soff, 0, 0);
        } else {
            const int soff = LAST ? 0 : TB::phase_bytes(k0, p.ldb);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(lds + (2 + buf) * TILE + TB::copy_dst(wave_u, j - A_COPIES)),
                16, (int)voff, soff, 0, 0);
        }
    };

    // Per-lane read bases in bytes for stage 0 of the tile at element `base`
    // (the wave's span starting at mn), four per factor: KC, base x serves
    // step x (row mn + l % 32, logical chunk 2 x + l / 32; fragment f adds 32
    // rows, 4096 bytes); MC, base x serves fragment x (k 0..3 of the lane
    // group at step 0; step s adds 16 rows, 8192 bytes, k 4..7 four rows,
    // 2048).  All the rest is an instruction offset.
    auto mc_elem = [](int r, int c) __attribute__((always_inline)) { return r * 256 + 8 * (c ^ (4 * (r & 3))); };
    auto frag_base = [&](auto kc, int base, int mn, int x) __attribute__((always_inline)) -> uint32_t {
        if constexpr (decltype(kc)::value) {
            return lds_addr(lds + base) + 2u * ((mn + li) * kBK + 8 * ((2 * x + lh) ^ sched_swz(li)));
        } else {
            const int n = mn + 32 * x + 16 * (tr_g & 1) + 4 * (tr_j & 3);
            const int row0 = 8 * (tr_g >> 1) + (tr_j >> 2);
            return lds_addr(lds + base) + 2u * (mc_elem(row0, n >> 3) + 4 * ((n >> 2) & 1));
        }
    };
    static_assert(kBK / 16 == 4 && FM == 4 && FN == 4, "four read bases per factor");
    uint32_t abase[4], bbase[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        abase[x] = frag_base(std::integral_constant<bool, KCA>{}, 0, wm * WM, x);
        bbase[x] = frag_base(std::integral_constant<bool, KCB>{}, 2 * TILE, wn * WN, x);
    }

    u32x4 a[2][FM], b[2][FN];
    // Read i (0 .. READS - 1) of one factor's fragments of step s into x: KC,
    // fragment i; MC, half i % 2 of fragment i / 2.
    auto read_one = [&](auto kc, u32x4 (&x)[4], const uint32_t (&base)[4], int s,
                        int i) __attribute__((always_inline)) {
        if constexpr (decltype(kc)::value) {
            x[i] = lds_read128(base[s] + 4096u * (uint32_t)i);
        } else {
            const int f = i / 2, r = i % 2;
            const u32x2 v = read_tr16_off(base[f], 8192 * s + 2048 * r);
            x[f][2 * r] = v[0];
            x[f][2 * r + 1] = v[1];
        }
    };
    // Read i of step s into set t, from the stage the bases point at: A's
    // reads first, then B's.
    auto read_op = [&](int s, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(std::integral_constant<bool, KCA>{}, a[t], abase, s, i);
        else read_one(std::integral_constant<bool, KCB>{}, b[t], bbase, s, i - TA::READS);
    };
    // Point the read bases at the other stage (from stage cur to cur ^ 1).
    auto flip_stage = [&](int cur) __attribute__((always_inline)) {
        const uint32_t d = cur ? (uint32_t)-32768 : 32768u;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            abase[x] += d;
            bbase[x] += d;
        }
    };
    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One step: the 16 matrix instructions on fragment set t (if MM); after
    // the q-th, reads 2q and 2q + 1 of step rs from stage rbuf into set t ^ 1
    // (if R) and, after each odd one, copy CB + q / 2 (while below CE) of the
    // phase at k_copy into stage cbuf (the last phase if lastc).
    auto step = [&](auto mm, int t, auto reads, int rs, auto cb, auto ce, int k_copy, int cbuf,
                    auto lastc) __attribute__((always_inline)) {
        constexpr bool MM = decltype(mm)::value;
        constexpr bool R = decltype(reads)::value;
        constexpr int CB = decltype(cb)::value, CE = decltype(ce)::value;
        unroll<FM * FN>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            if constexpr (MM) {
                acc[q / FN][q % FN] = mfma16<FMT>(a[t][q / FN], b[t][q % FN], acc[q / FN][q % FN]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (R && 2 * q < NREAD) {
                read_op(rs, t ^ 1, 2 * q);
                read_op(rs, t ^ 1, 2 * q + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q % 2 == 1 && CB + q / 2 < CE) {
                copy(CB + q / 2, k_copy, cbuf, lastc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    // The fragments of set t are complete (the tied wait also keeps the
    // compiler from adding a wait of its own that would cover later reads).
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        wait_tied(a[t]);
        wait_tied(b[t]);
    };
    // This wave's copies have landed; then the barrier makes every wave's
    // copies visible and releases the stage that was read.
    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        asm volatile("" ::: "memory");
    };
    using yes = std::true_type;
    using no = std::false_type;
    using c0 = std::integral_constant<int, 0>;
    using c8 = std::integral_constant<int, 8>;
    using c16 = std::integral_constant<int, 16>;
    // Steps 0..2 of the phase (step 0's fragments already read) and the wait
    // for step 3's; copies 8..15 of the phase at k_copy (the last phase if
    // lastc) into stage cbuf with step 0 if WC.
    auto steps012 = [&](auto wc, int k_copy, int cbuf, auto lastc) __attribute__((always_inline)) {
        constexpr bool WC = decltype(wc)::value;
        wait_set(0);
        if constexpr (WC) step(yes{}, 0, yes{}, 1, c8{}, c16{}, k_copy, cbuf, lastc);
        else step(yes{}, 0, yes{}, 1, c0{}, c0{}, 0, 0, no{});
        wait_set(1);
        step(yes{}, 1, yes{}, 2, c0{}, c0{}, 0, 0, no{});
        wait_set(0);
        step(yes{}, 0, yes{}, 3, c0{}, c0{}, 0, 0, no{});
        wait_set(1);
    };

    // Stage ph & 1 holds phase ph.  Between the barriers that end phases
    // ph - 1 and ph run the deferred last step of phase ph - 1 (with copies
    // 0..7 of phase ph + 1 and the first reads of phase ph, the read bases
    // already on its stage) and steps 0..2 of phase ph (copies 8..15 with
    // step 0).  The copies of phase P - 1 take the last phase's offsets: in
    // the prologue when P <= 2, else in the loop's final pass (peeled) and
    // the block after it.
    if (P == 1) {
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy(j, 0, 0, yes{});
    } else {
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy(j, 0, 0, no{});
    }
    barrier();
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(0, 0, i);
    if (P == 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) copy(j, kBK, 1, yes{});
    } else if (P > 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) copy(j, kBK, 1, no{});
    }
    __builtin_amdgcn_sched_barrier(0);
    int ph = 0;
    for (; ph + 3 < P; ++ph) {
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kBK, cur ^ 1, no{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(yes{}, 1, yes{}, 0, c0{}, c8{}, (ph + 2) * kBK, cur, no{});
    }
    if (ph + 2 < P) {                                       // copies 0..7 of the last phase
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kBK, cur ^ 1, no{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(yes{}, 1, yes{}, 0, c0{}, c8{}, (ph + 2) * kBK, cur, yes{});
        ++ph;
    }
    if (ph + 1 < P) {                                       // copies 8..15 of the last phase
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kBK, cur ^ 1, yes{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(yes{}, 1, yes{}, 0, c0{}, c0{}, 0, 0, no{});
        ++ph;
    }
    steps012(no{}, 0, 0, no{});
    step(yes{}, 1, no{}, 0, c0{}, c0{}, 0, 0, no{});

    // Guarded store (edge tiles run whole and store only what lies inside
    // C).  Register r of lane (li, lh) is row 8 (r / 4) + 4 lh + r % 4 of its
    // 32 x 32 block.
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

// ---------------------------------------------------------------------------
// op(A) x op(B): the backward-pass products (X^T dY, dY W^T) in mixed
// precision.  Each factor is an MN x K matrix of op(X) (MN = M for A, N for
// B) stored either
//   KC, k-contiguous (A as stored, B stored transposed): the LDS tile holds
//       MNT rows of 64 k (128 bytes), chunk c of row r at c ^ f(r), and a
//       lane's fragment is one 128-bit read, as for A in gemm16_kernel;
//   MC, mn-contiguous (B as stored, A stored transposed): the tile holds 64 k
//       rows of MNT values, chunk c of row r at c ^ 4 (r % 4), and a lane's
//       fragment is two ds_read_b64_tr_b16 reads, as for B in gemm16_kernel.
// Interior phases copy both tiles straight from global memory into LDS;
// ghost phases load chunk by chunk with zeros outside the matrix, into the
// same layout.  The k order (k = 16 s + 8 h + e for element e of lane half h
// in step s) does not depend on how a factor is stored, so every op pair
// gives the bits of gemm_mixed on explicitly transposed copies.
template <int MNT, bool KC, int NW>
struct Tile16 {
    static constexpr int ELEMS = MNT * kBK;                  // per stage
    static constexpr int CPR = KC ? kBK / 8 : MNT / 8;       // 16-byte chunks per stored row
    static constexpr int ROWS = KC ? MNT : kBK;              // stored rows per stage
    static constexpr int ROW_LEN = KC ? kBK : MNT;
    static constexpr int COPIES = ELEMS * 2 / 1024 / NW;     // direct 1 KB copies per wave
    static constexpr int ROWS_PER_COPY = 64 / CPR;
    static_assert(KC || (CPR >= 16 && 64 % CPR == 0), "mn-contiguous tile width");
    static_assert(COPIES * NW * 1024 == ELEMS * 2, "direct copy split");

    __device__ static int phys(int r, int c) { return KC ? (c ^ swz(r)) : (c ^ (4 * (r & 3))); }
    __device__ static int elem(int r, int c) { return r * ROW_LEN + 8 * phys(r, c); }
    // Global element offset of stored (row, col) of the tile at mn0, relative
    // to the phase's k0 (added separately: k0 for KC, k0 * ld for MC).
    __device__ static int64_t offset(int64_t ld, int mn0, int row, int col) {
        return KC ? (int64_t)(mn0 + row) * ld + col : (int64_t)row * ld + mn0 + col;
    }
    __device__ static int64_t phase_step(int64_t ld, int k0) { return KC ? (int64_t)k0 : (int64_t)k0 * ld; }
    // Eight stored values of (row, 8 c) with ghost zeros.
    template <bool VEC>
    __device__ static u32x4 ghost(const uint16_t* X, int64_t ld, int mn0, int mn_ext, int k0, int k_ext,
                                  int row, int c) {
        return KC ? load8_ghost<VEC>(X, mn0 + row, mn_ext, k0 + 8 * c, k_ext, ld)
                  : load8_ghost<VEC>(X, k0 + row, k_ext, mn0 + 8 * c, mn_ext, ld);
    }
    // Fragment of op(X) rows mb .. mb + 31, 16-deep step s (see gemm16_kernel).
    __device__ static u32x4 fragment(const uint16_t* t, int mb, int s, int lane) {
        if constexpr (KC) {
            return *reinterpret_cast<const u32x4*>(&t[elem(mb + (lane & 31), 2 * s + (lane >> 5))]);
        } else {
            const int g = lane >> 4, j = lane & 15;
            const int mn = mb + 16 * (g & 1) + 4 * (j & 3);
            u32x4 out;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int row = 16 * s + 8 * (g >> 1) + 4 * r + (j >> 2);
                const u32x2 v = read_tr16(lds_addr(t + elem(row, mn >> 3) + 4 * ((mn >> 2) & 1)));
                out[2 * r] = v[0];
                out[2 * r + 1] = v[1];
            }
            return out;
        }
    }
};

template <int FMT, int BM, int BN, int WAVES_M, int WAVES_N, bool KCA, bool KCB, bool VEC>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm16_op_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int FM = WM / 32, FN = WN / 32;
    using TA = Tile16<BM, KCA, NW>;
    using TB = Tile16<BN, KCB, NW>;
    constexpr int STAGE = TA::ELEMS + TB::ELEMS;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert((TA::ROWS * TA::CPR) % NT == 0 && (TB::ROWS * TB::CPR) % NT == 0, "ghost split");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;
    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;
    const bool fast_tile = VEC && (m0 + BM <= p.M) && (n0 + BN <= p.N);

    // direct copy j of this wave fills stored rows R .. R + ROWS_PER_COPY - 1,
    // R = ROWS_PER_COPY (wave + j NW); lane l writes physical chunk l % CPR of
    // row R + l / CPR, so it reads the logical chunk of that position
    int64_t a_doff[VEC ? TA::COPIES : 1], b_doff[VEC ? TB::COPIES : 1];
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < TA::COPIES; ++j) {
            const int row = TA::ROWS_PER_COPY * (wave_u + j * NW) + lane / TA::CPR;
            a_doff[j] = TA::offset(p.lda, m0, row, 8 * TA::phys(row, lane % TA::CPR));
        }
#pragma unroll
        for (int j = 0; j < TB::COPIES; ++j) {
            const int row = TB::ROWS_PER_COPY * (wave_u + j * NW) + lane / TB::CPR;
            b_doff[j] = TB::offset(p.ldb, n0, row, 8 * TB::phys(row, lane % TB::CPR));
        }
    }
    auto direct_tiles = [&](int k0, int buf) {
        if constexpr (VEC) {
            uint16_t* as = lds + buf * STAGE;
            uint16_t* bs = as + TA::ELEMS;
            const uint16_t* a = p.A + TA::phase_step(p.lda, k0);
            const uint16_t* b = p.B + TB::phase_step(p.ldb, k0);
#pragma unroll
            for (int j = 0; j < TA::COPIES; ++j)
                copy16_to_lds(a + a_doff[j], as + TA::ROWS_PER_COPY * (wave_u + j * NW) * TA::ROW_LEN);
#pragma unroll
            for (int j = 0; j < TB::COPIES; ++j)
                copy16_to_lds(b + b_doff[j], bs + TB::ROWS_PER_COPY * (wave_u + j * NW) * TB::ROW_LEN);
        }
    };
    // ghost phases: loaded and stored chunk by chunk (no registers held
    // across the math; these phases are rare in interior tiles)
    auto ghost_tiles_now = [&](int k0, int buf) {
        uint16_t* as = lds + buf * STAGE;
        uint16_t* bs = as + TA::ELEMS;
#pragma unroll
        for (int u = 0; u < TA::ROWS * TA::CPR / NT; ++u) {
            const int q = tid + u * NT, r = q / TA::CPR, c = q % TA::CPR;
            *reinterpret_cast<u32x4*>(&as[TA::elem(r, c)]) =
                TA::template ghost<VEC>(p.A, p.lda, m0, p.M, k0, p.K, r, c);
        }
#pragma unroll
        for (int u = 0; u < TB::ROWS * TB::CPR / NT; ++u) {
            const int q = tid + u * NT, r = q / TB::CPR, c = q % TB::CPR;
            *reinterpret_cast<u32x4*>(&bs[TB::elem(r, c)]) =
                TB::template ghost<VEC>(p.B, p.ldb, n0, p.N, k0, p.K, r, c);
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int s, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
#pragma unroll
        for (int f = 0; f < FM; ++f) a[f] = TA::fragment(as, wm * WM + f * 32, s, lane);
#pragma unroll
        for (int f = 0; f < FN; ++f) b[f] = TB::fragment(bs, wn * WN + f * 32, s, lane);
    };
    auto math = [&](int buf) {
        const uint16_t* as = lds + buf * STAGE;
        const uint16_t* bs = as + TA::ELEMS;
        u32x4 a[2][FM], b[2][FN];
        read_frags(as, bs, 0, a[0], b[0]);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            // this step's transposed reads were issued one step ago
            if constexpr (!KCA) wait_tied(a[s & 1]);
            if constexpr (!KCB) wait_tied(b[s & 1]);
            if (s + 1 < kBK / 16) read_frags(as, bs, s + 1, a[(s + 1) & 1], b[(s + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<FMT>(a[s & 1][i], b[s & 1][j], acc[i][j]);
        }
    };
    auto end_phase = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        asm volatile("" ::: "memory");
    };

    const int phases = ceil_div(p.K, kBK);
    const int full = fast_tile ? p.K / kBK : 0;       // phases copied straight (no ghosts)
    if (phases > 0) {
        if (full > 0) direct_tiles(0, 0);
        else ghost_tiles_now(0, 0);
    }
    end_phase();
    for (int ph = 0; ph < phases; ++ph) {
        const int cur = ph & 1, k_next = (ph + 1) * kBK;
        if (ph + 1 < full) direct_tiles(k_next, cur ^ 1);
        else if (ph + 1 < phases) ghost_tiles_now(k_next, cur ^ 1);
        // keep the next phase's copies ahead of the math
        __builtin_amdgcn_sched_barrier(0);
        math(cur);
        end_phase();
    }

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
using Launch16 = hipError_t (*)(const Gemm16Args&, hipStream_t, int, int, int, unsigned);

template <int FMT, int BM, int BN, int WAVES_M, int WAVES_N, bool DIRECT, bool VEC, bool BTR>
hipError_t launch16(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                    unsigned blocks) {
    hipLaunchKernelGGL((gemm16_kernel<FMT, BM, BN, WAVES_M, WAVES_N, DIRECT, VEC, BTR>), dim3(blocks),
                       dim3(WAVES_M * WAVES_N * 64), 0, s, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

struct MixedConfig {
    const char* name;
    int bm, bn, group_m;
    Launch16 launch[2][2];        // [format][vector loads]
};

// Misaligned operands use the element-wise kernel of the same tile shape
// (never direct copies).
#define MIXED(BM, BN, WM, WN, D, T)                                                                  \
    {{launch16<0, BM, BN, WM, WN, false, false, false>, launch16<0, BM, BN, WM, WN, D, true, T>},   \
     {launch16<1, BM, BN, WM, WN, false, false, false>, launch16<1, BM, BN, WM, WN, D, true, T>}}

// The scheduled kernel takes K a multiple of 8, an mn-contiguous factor's
// width (M for A stored transposed, N for B as stored) even,
// vector-aligned operands and operands below 2^31 bytes with a tile's
// overhang (its copies use 32-bit offsets); edge tiles run whole (see its
// descriptors).  Anything else runs the 8-wave kernel of the same tile
// (gemm16_kernel, configuration 6, or gemm16_op_kernel): same tiles, same k
// order, same bits.  op_a / op_b: 1 if that factor is stored transposed.
bool sched_fits(const Gemm16Args& p, int op_a, int op_b) {
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const bool widths = (op_a == 0 || p.M % 2 == 0) && (op_b != 0 || p.N % 2 == 0);
    return vec && widths && p.K % 8 == 0 && p.K > 0 && p.M > 0 && p.N > 0 &&
           2 * (a_rows + 256) * p.lda < (1ll << 31) && 2 * (b_rows + 256) * p.ldb < (1ll << 31);
}
template <int FMT, bool KCA, bool KCB>
hipError_t launch_sched_kernel(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                               unsigned blocks) {
    hipLaunchKernelGGL((gemm16_sched_kernel<FMT, KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}
// Tile-row groups: 4 for the scheduled kernel, 8 for the 8-wave kernel (each
// the fastest measured at 8192^3).
constexpr int kSchedGroupM = 4, kDirectGroupM = 8, kWide192GroupM = 4;
template <int FMT>
hipError_t launch_sched(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int /*group_m*/,
                        unsigned blocks) {
    if (!sched_fits(p, 0, 0))
        return launch16<FMT, 256, 256, 2, 4, true, true, true>(p, s, tiles_m, tiles_n, kDirectGroupM, blocks);
    return launch_sched_kernel<FMT, true, false>(p, s, tiles_m, tiles_n, kSchedGroupM, blocks);
}

// Configuration 9 (the k-split kernel, mfma16_ksplit.hip) where it takes
// the problem; other problems given to it run the 64 x 64 tiles of
// gemm16_kernel.
template <int FMT>
hipError_t launch_ksplit16_cfg(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                               unsigned blocks) {
    if (!ksplit16_fits(p, 0, 0))
        return launch16<FMT, 64, 64, 1, 2, false, true, false>(p, s, tiles_m, tiles_n, group_m, blocks);
    return launch_ksplit16(p, s, FMT, 0, 0);
}

// Configuration 12 (128 x 128 tiles whose four waves split the phases,
// mfma16_ksplit128.hip) where it takes the problem; else the 128 x 128
// tiles of configuration 7.
constexpr int kKsplit128GroupM = 8;
template <int FMT>
hipError_t launch_ksplit128_cfg(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                unsigned blocks) {
    if (!ksplit128_fits(p, 0, 0))
        return launch16<FMT, 128, 128, 2, 2, true, true, true>(p, s, tiles_m, tiles_n, group_m, blocks);
    return launch_ksplit128(p, s, FMT, 0, 0, kKsplit128GroupM);
}

// Configuration 10 (the scheduled kernel on v_mfma_f32_16x16x32,
// mfma16_wide.hip) where it takes the problem; else the 8-wave kernel, as
// for configuration 8 (its bits differ: another instruction).
template <int FMT>
hipError_t launch_wide_cfg(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int /*group_m*/,
                           unsigned blocks) {
    if (!wide_fits(p, 0, 0))
        return launch16<FMT, 256, 256, 2, 4, true, true, true>(p, s, tiles_m, tiles_n, kDirectGroupM, blocks);
    return launch_wide16(p, s, FMT, 0, 0, kSchedGroupM);
}

// Configuration 13 (the same kernel on 192 x 192 tiles) where it takes the
// problem; else the 8-wave kernel on 256 x 256 tiles, as configuration 10
// runs it (VEC: vector-aligned operands; the tile counts it is given are
// those of 192 x 192 tiles, so they are taken again for 256 x 256 ones).
template <int FMT, bool VEC>
hipError_t launch_wide192_cfg(const Gemm16Args& p, hipStream_t s, int /*tiles_m*/, int /*tiles_n*/,
                              int /*group_m*/, unsigned /*blocks*/) {
    if (VEC && wide_fits(p, 0, 0)) return launch_wide16_192(p, s, FMT, 0, 0, kWide192GroupM);
    const int tm = ceil_div(p.M, 256), tn = ceil_div(p.N, 256);
    const unsigned nb = (unsigned)((int64_t)tm * tn);
    if (VEC) return launch16<FMT, 256, 256, 2, 4, true, true, true>(p, s, tm, tn, kDirectGroupM, nb);
    return launch16<FMT, 256, 256, 2, 4, false, false, false>(p, s, tm, tn, kSchedGroupM, nb);
}

// Configuration 15 (the same kernel on 160 x 160 tiles), with the same
// fallback as configuration 13.
template <int FMT, bool VEC>
hipError_t launch_wide160_cfg(const Gemm16Args& p, hipStream_t s, int /*tiles_m*/, int /*tiles_n*/,
                              int /*group_m*/, unsigned /*blocks*/) {
    if (VEC && wide_fits(p, 0, 0)) return launch_wide16_160(p, s, FMT, 0, 0, kWide192GroupM);
    return launch_wide192_cfg<FMT, VEC>(p, s, 0, 0, 0, 0u);   // wide_fits fails there too
}

// Rows split (configuration 14): the first 256 m1 rows of op(A) -- whole
// tile rows filling all but the last round of 256 CUs -- on 256 x 256 tiles
// of the 16 x 16 x 32 scheduled kernel, the rest on 128 x 128 tiles whose
// four waves split the phases (if those are at most 256 and it takes the
// problem), else on 160 x 160 tiles if they need no more rounds of 256 CUs
// than 192 x 192 ones, else on 192 x 192 tiles; two launches in stream
// order, each part
// with the bits its kernel gives alone.  Where the 256 x 256 kernel does
// not take the problem, or there is no such split, configuration 10 runs
// the whole product.  op_a / op_b: 1 if that factor is stored transposed.
int rowsplit_rows(int M, int N) {
    const int64_t tm = ceil_div(M, 256), tn = ceil_div(N, 256);
    const int64_t rounds = (tm * tn + 255) / 256;
    const int64_t m1 = 256 * (rounds - 1) / tn;
    return (rounds >= 2 && m1 >= 1 && m1 < tm) ? (int)(256 * m1) : 0;
}
hipError_t launch_rowsplit(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b) {
    const int rows = rowsplit_rows(p.M, p.N);
    if (rows == 0 || !wide_fits(p, op_a, op_b)) return hipErrorNotSupported;
    Gemm16Args top = p, rest = p;
    top.M = rows;
    rest.M = p.M - rows;
    rest.A = p.A + (op_a ? (int64_t)rows : (int64_t)rows * p.lda);
    rest.C = p.C + (int64_t)rows * p.ldc;
    hipError_t e = launch_wide16(top, s, format, op_a, op_b, kSchedGroupM);
    if (e != hipSuccess) return e;
    const int64_t t128 = (int64_t)ceil_div(rest.M, 128) * ceil_div(rest.N, 128);
    if (t128 <= 256 && ksplit128_fits(rest, op_a, op_b))
        return launch_ksplit128(rest, s, format, op_a, op_b, kKsplit128GroupM);
    const int64_t r160 = ((int64_t)ceil_div(rest.M, 160) * ceil_div(rest.N, 160) + 255) / 256;
    const int64_t r192 = ((int64_t)ceil_div(rest.M, 192) * ceil_div(rest.N, 192) + 255) / 256;
    if (r160 <= r192) return launch_wide16_160(rest, s, format, op_a, op_b, kWide192GroupM);
    return launch_wide16_192(rest, s, format, op_a, op_b, kWide192GroupM);
}
template <int FMT>
hipError_t launch_rowsplit_cfg(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                               unsigned blocks) {
    if (rowsplit_rows(p.M, p.N) == 0 || !wide_fits(p, 0, 0)) return launch_wide_cfg<FMT>(p, s, tiles_m, tiles_n, group_m, blocks);
    return launch_rowsplit(p, s, FMT, 0, 0);
}

// Configuration 11 (the four-stage form, mfma16_wide4.hip) where it takes
// the problem; else the 8-wave kernel, as for configuration 8.
template <int FMT>
hipError_t launch_wide4_cfg(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int /*group_m*/,
                            unsigned blocks) {
    if (!sched_fits(p, 0, 0))
        return launch16<FMT, 256, 256, 2, 4, true, true, true>(p, s, tiles_m, tiles_n, kDirectGroupM, blocks);
    return launch_wide16_4stage(p, s, FMT, kSchedGroupM);
}

const MixedConfig kMixed[] = {
    {"mixed256x256_bk64_w2x4_directA", 256, 256, 8, MIXED(256, 256, 2, 4, true, false)},
    {"mixed256x256_bk64_w2x4", 256, 256, 8, MIXED(256, 256, 2, 4, false, false)},
    {"mixed128x128_bk64_w2x2", 128, 128, 8, MIXED(128, 128, 2, 2, false, false)},
    {"mixed64x64_bk64_w1x2", 64, 64, 8, MIXED(64, 64, 1, 2, false, false)},
    {"mixed256x256_bk64_w2x2_directA", 256, 256, 8, MIXED(256, 256, 2, 2, true, false)},
    {"mixed256x256_bk64_w2x2_directAB", 256, 256, 8, MIXED(256, 256, 2, 2, true, true)},
    {"mixed256x256_bk64_w2x4_directAB", 256, 256, 8, MIXED(256, 256, 2, 4, true, true)},
    {"mixed128x128_bk64_w2x2_directAB", 128, 128, 8, MIXED(128, 128, 2, 2, true, true)},
    // misaligned operands: the element-wise 8-wave kernel, as for 6
    {"mixed256x256_bk64_w4_sched", 256, 256, kSchedGroupM,
     {{launch16<0, 256, 256, 2, 4, false, false, false>, launch_sched<0>},
      {launch16<1, 256, 256, 2, 4, false, false, false>, launch_sched<1>}}},
    // four waves, each the whole 64 x 64 tile over every fourth phase;
    // misaligned operands: the element-wise 64 x 64 kernel
    {"mixed64x64_bk32_w4_ksplit", 64, 64, 8,
     {{launch16<0, 64, 64, 1, 2, false, false, false>, launch_ksplit16_cfg<0>},
      {launch16<1, 64, 64, 1, 2, false, false, false>, launch_ksplit16_cfg<1>}}},
    // the scheduled kernel's tiles on v_mfma_f32_16x16x32; misaligned
    // operands: the element-wise 8-wave kernel, as for 6
    {"mixed256x256_bk64_w4_wide", 256, 256, kSchedGroupM,
     {{launch16<0, 256, 256, 2, 4, false, false, false>, launch_wide_cfg<0>},
      {launch16<1, 256, 256, 2, 4, false, false, false>, launch_wide_cfg<1>}}},
    // the same with four 32-deep LDS stages (not picked by default)
    {"mixed256x256_bk32_w4_wide4stage", 256, 256, kSchedGroupM,
     {{launch16<0, 256, 256, 2, 4, false, false, false>, launch_wide4_cfg<0>},
      {launch16<1, 256, 256, 2, 4, false, false, false>, launch_wide4_cfg<1>}}},
    // four waves, each the whole 128 x 128 tile over every fourth phase;
    // misaligned operands: the element-wise 128 x 128 kernel
    {"mixed128x128_bk32_w4_ksplit", 128, 128, kKsplit128GroupM,
     {{launch16<0, 128, 128, 2, 2, false, false, false>, launch_ksplit128_cfg<0>},
      {launch16<1, 128, 128, 2, 2, false, false, false>, launch_ksplit128_cfg<1>}}},
    // configuration 10's kernel on 192 x 192 tiles; misaligned operands: the
    // element-wise 8-wave kernel on 256 x 256 tiles, as for 6
    {"mixed192x192_bk64_w4_wide", 192, 192, kWide192GroupM,
     {{launch_wide192_cfg<0, false>, launch_wide192_cfg<0, true>},
      {launch_wide192_cfg<1, false>, launch_wide192_cfg<1, true>}}},
    // the rows of all but the last round of 256 x 256 tiles on them, the rest
    // on k-split 128 x 128 or on 192 x 192 tiles; misaligned operands: the
    // element-wise 8-wave kernel, as for 6
    {"mixed256x256_rowsplit", 256, 256, kSchedGroupM,
     {{launch16<0, 256, 256, 2, 4, false, false, false>, launch_rowsplit_cfg<0>},
      {launch16<1, 256, 256, 2, 4, false, false, false>, launch_rowsplit_cfg<1>}}},
    // configuration 10's kernel on 160 x 160 tiles; misaligned operands: the
    // element-wise 8-wave kernel on 256 x 256 tiles, as for 13
    {"mixed160x160_bk64_w4_wide", 160, 160, kWide192GroupM,
     {{launch_wide160_cfg<0, false>, launch_wide160_cfg<0, true>},
      {launch_wide160_cfg<1, false>, launch_wide160_cfg<1, true>}}},
};
#undef MIXED
constexpr int kNumMixed = (int)(sizeof(kMixed) / sizeof(kMixed[0]));
constexpr int kKsplitConfig = 9;          // mixed64x64_bk32_w4_ksplit
constexpr int kWideConfig = 10;           // mixed256x256_bk64_w4_wide
constexpr int kKsplit128Config = 12;      // mixed128x128_bk32_w4_ksplit
constexpr int kWide192Config = 13;        // mixed192x192_bk64_w4_wide
constexpr int kRowsplitConfig = 14;       // mixed256x256_rowsplit
constexpr int kWide160Config = 15;        // mixed160x160_bk64_w4_wide

// op kernels, chosen by tile, op pair and load path
template <int FMT, int BM, int BN, int WM, int WN, bool KCA, bool KCB, bool VEC>
hipError_t launch16_op(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                       unsigned blocks) {
    hipLaunchKernelGGL((gemm16_op_kernel<FMT, BM, BN, WM, WN, KCA, KCB, VEC>), dim3(blocks), dim3(WM * WN * 64),
                       0, s, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}
template <int FMT, int BM, int BN, int WM, int WN>
Launch16 op_launcher(int op_a, int op_b, bool vec) {
    // op 0 = factor as stored: A k-contiguous, B mn-contiguous; op 1 the reverse
    const int key = 4 * op_a + 2 * op_b + (vec ? 1 : 0);
    switch (key) {
        case 0: return launch16_op<FMT, BM, BN, WM, WN, true, false, false>;
        case 1: return launch16_op<FMT, BM, BN, WM, WN, true, false, true>;
        case 2: return launch16_op<FMT, BM, BN, WM, WN, true, true, false>;
        case 3: return launch16_op<FMT, BM, BN, WM, WN, true, true, true>;
        case 4: return launch16_op<FMT, BM, BN, WM, WN, false, false, false>;
        case 5: return launch16_op<FMT, BM, BN, WM, WN, false, false, true>;
        case 6: return launch16_op<FMT, BM, BN, WM, WN, false, true, false>;
        default: return launch16_op<FMT, BM, BN, WM, WN, false, true, true>;
    }
}
}  // namespace

// op(A) x op(B): the tiles gemm_mixed picks -- 256 x 256 (the scheduled
// kernel on v_mfma_f32_16x16x32, mfma16_wide.hip, where it fits, else eight
// waves of gemm16_op_kernel) or 192 x 192 (the same kernel) once there are
// 128 tiles of 256, else the k-split kernels, 192 x 192 tiles or 128 x 128
// tiles of four waves, or 160 x 160 tiles; where the 192 x 192, 160 x 160 or
// k-split kernels do not fit,
// the 256 x 256 or 128 x 128 tiles by the same count.  A and B are the stored matrices; vector loads (and
// the direct copies) need 4-byte aligned bases and even leading dimensions,
// as for gemm_mixed.
hipError_t launch_mixed_op(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b) {
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int64_t t256 = (int64_t)ceil_div(p.M, 256) * ceil_div(p.N, 256);
    const int pick = mixed_pick_config(p.M, p.N, p.K);
    if (pick == kKsplitConfig && ksplit16_fits(p, op_a, op_b)) return launch_ksplit16(p, s, format, op_a, op_b);
    if (pick == kKsplit128Config && ksplit128_fits(p, op_a, op_b))
        return launch_ksplit128(p, s, format, op_a, op_b, kKsplit128GroupM);
    if (pick == kWide192Config && wide_fits(p, op_a, op_b))
        return launch_wide16_192(p, s, format, op_a, op_b, kWide192GroupM);
    if (pick == kWide160Config && wide_fits(p, op_a, op_b))
        return launch_wide16_160(p, s, format, op_a, op_b, kWide192GroupM);
    if (pick == kRowsplitConfig && rowsplit_rows(p.M, p.N) > 0 && wide_fits(p, op_a, op_b))
        return launch_rowsplit(p, s, format, op_a, op_b);
    const bool big = t256 >= 128;
    const int tile = big ? 256 : 128;
    const int tiles_m = ceil_div(p.M, tile), tiles_n = ceil_div(p.N, tile);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (big && wide_fits(p, op_a, op_b)) return launch_wide16(p, s, format, op_a, op_b, kSchedGroupM);
    Launch16 fn;
    if (big) fn = format ? op_launcher<1, 256, 256, 2, 4>(op_a, op_b, vec) : op_launcher<0, 256, 256, 2, 4>(op_a, op_b, vec);
    else fn = format ? op_launcher<1, 128, 128, 2, 2>(op_a, op_b, vec) : op_launcher<0, 128, 128, 2, 2>(op_a, op_b, vec);
    return fn(p, s, tiles_m, tiles_n, kDirectGroupM, (unsigned)blocks);
}

int mixed_num_configs() { return kNumMixed; }
const char* mixed_config_name(int c) { return (c >= 0 && c < kNumMixed) ? kMixed[c].name : nullptr; }

// 256 x 256 tiles on the scheduled kernel of the 16 x 16 x 32 instruction
// (configuration 10, which itself runs configuration 6 on problems it does
// not take) from 128 of them, half the CUs: measured, 144 such tiles
// (3072^3) still beat 576 of 128 x 128 by 40 %; at 8192^3 it runs bf16 at
// 1395 TFLOP/s against 1332 for the 32 x 32 x 16 form (configuration 8) on
// the same box, f16 at 1340 against 1250.  There, 192 x 192 tiles of the
// same kernel (configuration 13; K even) where they need fewer rounds of
// 256 CUs by the measured cost of a 192 tile, 0.8 of a 256 tile per phase
// (its copies, 48 KB per 64-deep phase, take longer than its matrix
// instructions): 4 rounds of 192 < 5 rounds of 256 (bf16: 3072^3 1169
// against 944 TFLOP/s, 4100^2 x 4096 1078 against 830, 2048 x 4096 x 1024
// 709 against 581; 3584^3, one round of 256 against two of 192, 1278
// against 893).  Else, with K a multiple of 8 and the last round of 256 x
// 256 tiles under 40 % full, the rows split (configuration 14): 4352^3 1173
// against 955, 4608^3 1170 against 1074, 7168^3 1373 against 1253, 8200^2 x
// 4096 1303 against 1254, 4000 x 5000 x 4096 1079 against 996 (6144^3 1219
// against 1266: the one loss measured).  Else, below
// 128 tiles of 128 x 128 and with K a multiple of 8, 64 x 64 tiles whose
// four waves split the phases (mfma16_ksplit.hip; measured bf16: 1024^2 x
// 4096 479 against 186 TFLOP/s on the 128 x 128 tiles, 1000^3 234 against
// 53, 1024^3 297 against 160; 1536^3, with 144 tiles of 128 x 128, 321
// against 339).  Else, with at most 256 tiles of 128 x 128 (one per CU) and
// K of at least 1024 (a multiple of 8), 128 x 128 tiles whose four waves
// split the phases (mfma16_ksplit128.hip; measured bf16: 2048^3 697 against
// 586 TFLOP/s on the 128 x 128 tiles with direct copies, 1536^3 355 against
// 344; with 400 tiles (2560^3) or K = 256 they lose).  Else, with at least
// 140 tiles of 192 x 192 (more than half a round; K even), those tiles
// (bf16: 2816^3 967 against 847 on 128 x 128 tiles, 2560^3 798 against 764,
// 2048 x 3072 x 512 408 against 385; with 132 (1024 x 4096 x 1024) 410
// against 476); and with K % 8 != 0 (even) from 32 of them if K is below
// 1536, or, with fewer than 128 tiles of 128 x 128, K % 4 = 2 (the 128 x
// 128 and 64 x 64 tiles then run without direct copies, and with K % 4 = 2
// element by element: 1000 x 2000 x 500 145 against 94, 1500 x 3000 x 700
// 331 against 185, 1000^2 x 2002 102 against 50 on 64 x 64 tiles, 800 x
// 1200 x 3002 105 against 50; 1536^2 x 1538 244 against 274, 1024^2 x 4092
// 129 against 155).  Wherever 192 x 192 tiles are chosen, 160 x 160 ones
// (configuration 15) if they need no more rounds of 256 CUs: a round of
// them is the cheaper, its tiles having 0.69 of the area (bf16: 2560^3 861
// against 796 TFLOP/s, 2304^3 707 against 660, 1280 x 5120 x 2048 834
// against 780, 2560^2 x 1024 655 against 602; with one round more they lose:
// 2816^3 590 against 988, 2048 x 4096 x 1024 500 against 724).  Else 128 x 128 tiles with
// both factors copied straight into LDS from 128 of them (64 for K of at
// least 2048), else 64 x 64 tiles.
int mixed_pick_config(int M, int N, int K) {
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t192 = (int64_t)ceil_div(M, 192) * ceil_div(N, 192);
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    const bool even_k = K > 0 && K % 2 == 0;
    const int64_t t160 = (int64_t)ceil_div(M, 160) * ceil_div(N, 160);
    const int64_t r256 = (t256 + 255) / 256, r192 = (t192 + 255) / 256;   // rounds of 256 CUs
    const int64_t r160 = (t160 + 255) / 256;
    const int narrow = r160 <= r192 ? kWide160Config : kWide192Config;    // where 192 tiles win
    if (t256 >= 128) {
        if (even_k && 4 * r192 < 5 * r256) return narrow;
        const int64_t last = t256 - 256 * (r256 - 1);      // tiles in the last round
        return K % 8 == 0 && 5 * last < 2 * 256 && rowsplit_rows(M, N) > 0 ? kRowsplitConfig : kWideConfig;
    }
    if (t128 < 128 && K % 8 == 0 && K > 0) return kKsplitConfig;
    if (t128 <= 256 && K >= 1024 && K % 8 == 0) return kKsplit128Config;
    const bool ragged_k = K % 8 != 0 && t192 >= 32 && (K < 1536 || (t128 < 128 && K % 4 == 2));
    if (even_k && (t192 >= 140 || ragged_k)) return narrow;
    if (t128 >= 128 || (t128 >= 64 && K >= 2048)) return 7;
    return 3;
}

// hipErrorInvalidValue: the grid would exceed the launch limits.
hipError_t launch_mixed(const Gemm16Args& p, hipStream_t s, int format, int config) {
    const MixedConfig& c = kMixed[(config >= 0 && config < kNumMixed) ? config : 0];
    // vector loads: 4-byte aligned bases and even leading dimensions
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int tiles_m = ceil_div(p.M, c.bm), tiles_n = ceil_div(p.N, c.bn);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    return c.launch[format ? 1 : 0][vec ? 1 : 0](p, s, tiles_m, tiles_n, c.group_m, (unsigned)blocks);
}

}  // namespace gemmf32
