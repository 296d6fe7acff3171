// mfma16_wide4.hip -- the 16 x 16 x 32 scheduled 256 x 256 mixed-precision
// kernel with four 32-deep LDS stages (configuration
// mixed256x256_bk32_w4_wide4stage; gemm_mixed picks the two-stage form of
// mfma16_wide.hip).
//
// The one-volume PMPP notes run the fully connected layer as a matrix
// product on matrix units fed FP16 or BF16 and accumulating in FP32
// (deep-learning chapter, "FC Layer = GEMM", "Mixed Precision"); this is
// that product with the tiled structure of the pages' shared-memory chapter
// (tiles staged in LDS, ghost zeros past the matrix edges, a guarded store).
//
// 256 x 256 tiles, four waves (one per SIMD) of 128 x 128 each, 8 x 8 blocks
// of 16 x 16 per wave; 32-deep phases of 64 matrix instructions per wave;
// four LDS stages; every instruction of the K loop placed in program order.
// During phase ph a wave runs its 64 instructions on fragments read during
// phase ph - 1, reads the fragments of phase ph + 1 (one read after each of
// the first instructions), and copies its eighth of phase ph + 4 into the
// stage phase ph has just left (one copy after every eighth instruction);
// between phases it waits for its reads, for the copies of phase ph + 2
// (those of the next two phases stay in flight) and for the other waves.
// Against the two-stage form (one barrier per 64 k, copies one phase ahead
// in the second 32-k step) a copy has two to three phases to land instead
// of one and the copies spread over every phase, at the cost of a barrier
// per 32 k: measured on one MI355X, bf16, against the two-stage form,
// 8192^3 1449 against 1431 TFLOP/s (its copy waits fall from 4-7 % of the
// time to 0.6 %), but 4096^3 1362 against 1434 and 2048 x 8192 x 4096 1331
// against 1399 (one round of tiles, where the latency was already hidden).
// The 16-bit product needs 32 bytes per clock per CU from L2 at full
// matrix rate, about what the L2 delivers into LDS under load (measured:
// 32.5 bytes per clock per CU), so the copies' timing matters.  The stage of
// each phase is an instruction offset (the loop is unrolled by the four
// stages), so the loop holds no vector ALU instruction besides the matrix
// instructions.
//
// Tiles (per stage; 64 banks of 4 bytes; a 128-bit read serves, per
// half-wave, the 4-lane quads of even index parity in one cycle and the
// others in the next; 64-bit reads serve 32 lanes a cycle):
//   KC (k-contiguous factor: A as stored, B stored transposed): 256 rows of
//      32 k (64 bytes), 16-byte chunk c (8 k) of row r at c ^ (2 ((r / 8) mod
//      2)); a fragment (16 rows, 32 k) is one 128-bit read of row 16 f +
//      l % 16, chunk l / 16, conflict free; a 1 KB copy fills 16 rows.
//   MC (mn-contiguous factor: B as stored, A stored transposed): 16 pairs
//      of 512-byte k rows, pair m at byte 1056 m (32 bytes of padding after
//      each); k row kappa of the phase (kappa = 8 g + 4 h + e: lane group g,
//      read h, e = 0..3) is row h of pair e + 4 g and holds the tile's 256
//      values in order; a fragment is two ds_read_b64_tr_b16 reads (h = 0,
//      1) whose 32 lanes a cycle read 8 rows in pairs 8 banks apart; a 1 KB
//      copy fills one pair.
// One per-lane read base per factor serves every fragment, read and stage.
// Stage sizes 16384 (KC) and 16896 (MC) bytes: at most 135168 bytes of LDS.
//
// Edges: each buffer descriptor ends at its stored matrix's last element,
// and a copy that must bring zeros has a per-lane offset past that end by
// itself (rows of a KC factor past the tile's edge in every phase; lanes at
// k >= K, which only the prologue's phases hold).  The column overhang of
// an MC factor reads the next row (only C entries outside the matrix use
// it), or, in its last row (also a prologue phase, scalar offset 0), its
// dwords up to the descriptor's end and zeros past it.
//
// The k order inside each instruction (k = 32 b + 8 (l / 16) + e of lane l
// in block b) and the order of the blocks do not depend on how a factor is
// stored, so the four op pairs give the same bits on explicitly transposed
// copies.
#include "mfma16_common.h"

namespace gemmf32 {

namespace {

struct Wide4TileKC {
    static constexpr bool IS_KC = true;
    static constexpr int STAGE_BYTES = 16384;
    static constexpr int READS = 8;                       // LDS reads per phase (8 fragments)
    __host__ __device__ static constexpr int swz(int r) { return ((r >> 3) & 1) << 1; }
    // Copy j (0..3) of wave w fills stage bytes 1024 q .. + 1023, q = w + 4 j:
    // rows 16 q .. + 15; lane l fills physical chunk l % 4 of row 16 q + l / 4.
    __host__ __device__ static int copy_q(int w, int j) { return w + 4 * j; }
    __host__ __device__ static int copy_dst(int w, int j) { return 1024 * copy_q(w, j); }
    __host__ __device__ static int copy_row(int w, int j, int lane) { return 16 * copy_q(w, j) + lane / 4; }
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        return 8 * ((lane % 4) ^ swz(copy_row(w, j, lane)));
    }
    __host__ __device__ static int copy_mn(int w, int j, int lane) { return copy_row(w, j, lane); }
    __host__ __device__ static int64_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        return 2 * ((int64_t)(mn0 + copy_row(w, j, lane)) * ld + copy_k(w, j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return 2 * (int64_t)k0; }
    __host__ __device__ static uint32_t read_base(int lane, int mn) {
        return (uint32_t)(64 * (mn + lane % 16) + 16 * ((lane / 16) ^ swz(lane % 16)));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int f, int h) { return 1024u * f + 0u * h; }
};

struct Wide4TileMC {
    static constexpr bool IS_KC = false;
    static constexpr int STAGE_BYTES = 16 * 1056;
    static constexpr int READS = 16;                      // LDS reads per phase (8 fragments x 2)
    __host__ __device__ static int copy_q(int w, int j) { return w + 4 * j; }
    __host__ __device__ static int copy_dst(int w, int j) { return 1056 * copy_q(w, j); }
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        const int q = copy_q(w, j);
        return 8 * ((q >> 2) & 3) + 4 * (lane / 32) + (q & 3);
    }
    __host__ __device__ static int copy_mn(int w, int j, int lane) { return 8 * (lane % 32); }
    __host__ __device__ static int64_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        return 2 * ((int64_t)copy_k(w, j, lane) * ld + mn0 + copy_mn(w, j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return 2 * (int64_t)k0 * ld; }
    __host__ __device__ static uint32_t read_base(int lane, int mn) {
        const int j = lane % 16, g = lane / 16;
        return (uint32_t)(1056 * (j / 4 + 4 * g) + 2 * (mn + 4 * (j % 4)));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int f, int h) { return 32u * f + 512u * h; }
};

template <bool KC>
using Wide4Tile = std::conditional_t<KC, Wide4TileKC, Wide4TileMC>;

template <int FMT, bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm16_wide4_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    constexpr int BM = 256, BN = 256, WM = 128, WN = 128, BK = 32, FM = 8, FN = 8, NS = 4;
    using TA = Wide4Tile<KCA>;
    using TB = Wide4Tile<KCB>;
    constexpr int SA = TA::STAGE_BYTES, SB = TB::STAGE_BYTES;
    constexpr int A_COPIES = 4, NCOPY = 8;                // 1 KB copies per wave and phase
    constexpr int NREAD = TA::READS + TB::READS;          // LDS reads per phase
    static_assert(NREAD <= 32, "one read per matrix instruction, in the first half of a phase");
    __shared__ __attribute__((aligned(16))) unsigned char lds[NS * (SA + SB)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave_u / 2, wn = wave_u % 2;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        doff[j] = (uint32_t)TA::copy_src(wave_u, j, lane, m0, p.lda);
        doff[A_COPIES + j] = (uint32_t)TB::copy_src(wave_u, j, lane, n0, p.ldb);
    }
    constexpr int kRawBufferWord3 = 0x00020000;
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.A), (short)0, (int)(2 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.B), (short)0, (int)(2 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    // The K range splits into KB = ceil(K / 32) blocks of 32 k (block b at k
    // = 32 b; the last one may reach past K, a multiple of 8).  The phases,
    // P of them, a multiple of NS, take the blocks in this order: the last
    // block, then Z = P - KB phases of zeros (+0 products: an accumulator
    // that starts at +0 keeps its bits), then blocks 0, 1, ..., KB - 2.  So
    // phases 0 .. 3, copied in the prologue with the block folded into each
    // lane's offset (lanes at k >= K, and a zero phase's lanes, past the
    // end), hold the last block -- every k >= K and an mn-contiguous
    // factor's last row -- and every later phase is an interior block whose
    // lanes are in range, or past the end by their own offset, with the
    // phase in the scalar offset.
    const int KB = ceil_div(p.K, BK);
    const int P = NS * ceil_div(KB, NS);
    const int Z = P - KB;
    constexpr uint32_t kPastEnd = 0x80000000u;
    auto copy_at = [&](int j, uint32_t voff, int soff, int stage) __attribute__((always_inline)) {
        if (j < A_COPIES) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(lds + stage * SA + TA::copy_dst(wave_u, j)), 16,
                (int)voff, soff, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(lds + NS * SA + stage * SB + TB::copy_dst(wave_u, j - A_COPIES)),
                16, (int)voff, soff, 0, 0);
        }
    };
    // Scalar offsets of the phase at position ph >= NS (block ph - Z - 1);
    // past the last phase, 0: the copy then brings block-0 rows into a stage
    // no wave reads again (every lane in range or past the end by its own
    // offset).
    auto soff_a = [&](int ph) __attribute__((always_inline)) {
        return ph < P ? (int)TA::phase_bytes(BK * (ph - Z - 1), p.lda) : 0;
    };
    auto soff_b = [&](int ph) __attribute__((always_inline)) {
        return ph < P ? (int)TB::phase_bytes(BK * (ph - Z - 1), p.ldb) : 0;
    };
    // Phase s < NS into stage s, the block folded into each lane's offset.
    auto copy_first = [&](int s) __attribute__((always_inline)) {
        const bool zeros = s >= 1 && s <= Z;
        const int k0 = s == 0 ? BK * (KB - 1) : BK * (s - Z - 1);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) {
            const int kl = j < A_COPIES ? TA::copy_k(wave_u, j, lane) : TB::copy_k(wave_u, j - A_COPIES, lane);
            const int64_t pb = j < A_COPIES ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb);
            copy_at(j, !zeros && k0 + kl < p.K ? (uint32_t)((int64_t)doff[j] + pb) : kPastEnd, 0, s);
        }
    };

    // Opaque to the compiler, so that it keeps each factor's reads on its own
    // base with the stage and fragment as instruction offsets (B's base lies
    // more than 2^16 bytes past A's, out of an offset's reach).
    uint32_t abase = lds_addr(lds) + TA::read_base(lane, wm * WM);
    uint32_t bbase = lds_addr(lds) + NS * SA + TB::read_base(lane, wn * WN);
    asm volatile("" : "+v"(abase), "+v"(bbase));

    u32x4 aq[2][FM], bq[2][FN];
    u32x2 ah[2][FM][2], bh[2][FN][2];
    auto read_one = [&](auto tile, u32x4 (&q)[8], u32x2 (&hv)[8][2], uint32_t base, auto stg, int i)
                        __attribute__((always_inline)) {
        using T = decltype(tile);
        constexpr uint32_t SOFF = (uint32_t)T::STAGE_BYTES * decltype(stg)::value;
        if constexpr (T::IS_KC) q[i] = lds_read128(base + SOFF + T::read_imm(i, 0));
        else hv[i / 2][i % 2] = read_tr16_off(base, (int)(SOFF + T::read_imm(i / 2, i % 2)));
    };
    // With both factors k-contiguous, B's 128-bit fragments are also held
    // as halves (as 128-bit values beside A's the allocator moved the
    // accumulators every trip).
    constexpr bool B_HALVES = KCA && KCB;
    auto read_op = [&](auto stg, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) {
            read_one(TA{}, aq[t], ah[t], abase, stg, i);
        } else if constexpr (B_HALVES) {
            constexpr uint32_t SOFF = (uint32_t)TB::STAGE_BYTES * decltype(stg)::value;
            const u32x4 v = lds_read128(bbase + SOFF + TB::read_imm(i - TA::READS, 0));
            bh[t][i - TA::READS][0] = u32x2{v[0], v[1]};
            bh[t][i - TA::READS][1] = u32x2{v[2], v[3]};
        } else {
            read_one(TB{}, bq[t], bh[t], bbase, stg, i - TA::READS);
        }
    };
    auto frag_a = [&](int t, int i) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCA) return aq[t][i];
        else return u32x4{ah[t][i][0][0], ah[t][i][0][1], ah[t][i][1][0], ah[t][i][1][1]};
    };
    auto frag_b = [&](int t, int j) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCB && !B_HALVES) return bq[t][j];
        else return u32x4{bh[t][j][0][0], bh[t][j][0][1], bh[t][j][1][0], bh[t][j][1][1]};
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        if constexpr (KCA) wait_tied(aq[t]);
        else wait_tied(ah[t]);
        if constexpr (KCB && !B_HALVES) wait_tied(bq[t]);
        else wait_tied(bh[t]);
    };
    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Phase ph in stage U = ph % NS, fragments in set U % 2: its 64 matrix
    // instructions; after instruction q (q < NREAD) read q of phase ph + 1
    // (from stage (U + 1) % NS; past the last phase these reads are never
    // used), and after every eighth the copy q / 8 of phase ph + 4 into stage
    // U (whose fragments were read during phase ph - 1).
    auto phase = [&](auto uc, int ph) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        constexpr int T = U & 1;
        using NEXT = std::integral_constant<int, (U + 1) % NS>;
        const int sa = soff_a(ph + 4), sb = soff_b(ph + 4);
        unroll<FM * FN>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            acc[q / FN][q % FN] = mfma16x16<FMT>(frag_a(T, q / FN), frag_b(T, q % FN), acc[q / FN][q % FN]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (q < NREAD) {
                read_op(NEXT{}, T ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q % 8 == 7) {
                constexpr int j = q / 8;
                copy_at(j, doff[j], j < A_COPIES ? sa : sb, U);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    // Between phases: the fragments of the phase just run stay live up to
    // here (the allocator otherwise hands their registers to the next set
    // early and must move values at the loop's back edge); this wave's reads
    // of the next phase are done and the copies of the phase after it have
    // landed (the 16 of the two phases after that may still be in flight);
    // then the barrier (a bare s_barrier: the compiler would wait for every
    // copy before a fenced one).
    auto sync = [&](auto uc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        if constexpr (KCA) keep_alive(aq[U & 1]);
        else keep_alive(ah[U & 1]);
        if constexpr (KCB && !B_HALVES) keep_alive(bq[U & 1]);
        else keep_alive(bh[U & 1]);
        wait_set((U & 1) ^ 1);
        asm volatile("s_waitcnt vmcnt(16)\n s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: phases 0 .. 3 in flight; phases 0 and 1 landed; phase 0's
    // fragments read; a second barrier so that no wave copies into stage 0
    // before all have read it.
#pragma unroll
    for (int s = 0; s < NS; ++s) copy_first(s);
    asm volatile("s_waitcnt vmcnt(16)\n s_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(std::integral_constant<int, 0>{}, 0, i);
    wait_set(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // The phase loop, unrolled by the NS stages (P is a multiple of NS; the
    // sync after the last phase only waits).
    for (int ph0 = 0; ph0 < P; ph0 += NS) {
        unroll<NS>([&](auto uc) __attribute__((always_inline)) {
            phase(uc, ph0 + decltype(uc)::value);
            sync(uc);
        });
    }
    // no copy may still be writing LDS when the workgroup ends
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    const int row0 = m0 + wm * WM + 4 * (lane >> 4), col0 = n0 + wn * WN + (lane & 15);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 16 * i + r;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = col0 + 16 * j;
                if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = acc[i][j][r];
            }
        }
}

template <int FMT, bool KCA, bool KCB>
hipError_t launch_wide4_kernel(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                              unsigned blocks) {
    hipLaunchKernelGGL((gemm16_wide4_kernel<FMT, KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

}  // namespace

// A k-contiguous (as stored), B mn-contiguous (as stored); format 0
// bfloat16, 1 binary16.  The caller checks that the problem fits (the
// scheduled kernels' conditions).
hipError_t launch_wide16_4stage(const Gemm16Args& p, hipStream_t s, int format, int group_m) {
    const int tiles_m = ceil_div(p.M, 256), tiles_n = ceil_div(p.N, 256);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    return format ? launch_wide4_kernel<1, true, false>(p, s, tiles_m, tiles_n, group_m, (unsigned)blocks)
                  : launch_wide4_kernel<0, true, false>(p, s, tiles_m, tiles_n, group_m, (unsigned)blocks);
}

}  // namespace gemmf32
