// mfma16_wide.hip -- the scheduled 256 x 256 mixed-precision kernel
// (bfloat16 or binary16 factors, binary32 accumulation) on the 16 x 16 x 32
// matrix instruction.
//
// The one-volume PMPP notes run the fully connected layer as a matrix
// product on matrix units fed FP16 or BF16 and accumulating in FP32
// (deep-learning chapter, "FC Layer = GEMM", "Mixed Precision"); this is
// that product with the tiled structure of the pages' shared-memory chapter
// (tiles staged in LDS, ghost zeros past the matrix edges, a guarded store).
//
// Same block structure as gemm16_sched_kernel (mfma16.hip): 256 x 256 tiles,
// four waves (one per SIMD) of 128 x 128 each, 64-deep phases in two LDS
// stages, one barrier per phase, every instruction of the K loop placed in
// program order.  The instruction is v_mfma_f32_16x16x32 instead of
// 32 x 32 x 16: a wave's tile is 8 x 8 blocks of 16 x 16 and a phase is two
// 32-deep steps of 64 instructions (the same matrix-core clocks).  In a bare
// loop this form sustains a higher clock on MI355X than 32 x 32 x 16.
//
// The same kernel runs 192 x 192 tiles (template parameter BT): waves of 96
// x 96 (6 x 6 blocks), steps of 36 instructions, 6 copies per wave and phase
// for a k-contiguous factor (rows 0..191 of the layout below) and 8 for an
// mn-contiguous one (the layout below with each 512-byte k-row slot holding
// 192 values, the lanes of values 192..255 copying zeros).  Its copies need
// 42.7 bytes per clock per CU at the full matrix rate against 32 for 256 x
// 256 tiles: it is chosen only where its tile count fills the rounds of 256
// CUs much better.  Likewise 160 x 160 tiles: waves of 80 x 80 (5 x 5
// blocks), steps of 25 instructions, 5 copies per wave and phase for a
// k-contiguous factor and 8 for an mn-contiguous one (lanes of values
// 160..255 copying zeros); 51.2 bytes per clock per CU at the full matrix
// rate.
//
// The LDS tiles are laid out so that at most two per-lane bases per factor
// serve every fragment, step and read of a phase (all the rest are
// instruction offsets), and both kinds read without bank conflicts (64 banks
// of 4 bytes; measured):
//   KC (k-contiguous factor: A as stored, B stored transposed): 256 rows of
//      64 k (128 bytes), 16-byte chunk c (8 k) of row r at c ^ ((r / 2) mod
//      8), as in gemm16_sched_kernel.  A fragment (16 rows, 32 k) is one
//      128-bit read of row 16 f + l % 16, chunk 4 s + l / 16; the swizzle
//      depends on l % 16 only, so each step has one base and fragment f is
//      an instruction offset.  A 1 KB copy fills 8 rows.  (Rows of 32 k, 64
//      bytes, read this way conflict 2-way on gfx950 under every lane-to-
//      cycle grouping of 128-bit reads that agrees with the measured
//      conflict counts: the hardware does not serve lanes 0-15, 16-31, ...
//      together.)
//   MC (mn-contiguous factor: B as stored, A stored transposed): the stage is
//      32 pairs of 512-byte k rows, pair m at byte 1056 m (32 bytes of padding
//      after each pair); k row kappa of the phase (kappa = 32 s + 8 g + 4 h +
//      e: step s, lane group g, read h, e = 0..3) is row h of pair
//      e + 4 g + 16 s and holds the tile's 256 values in order.  A fragment
//      is two ds_read_b64_tr_b16 reads (h = 0, 1); the 8 rows one cycle reads
//      lie in pairs whose m mod 8 differ, each pair shifted by 8 banks
//      against the last.  A 1 KB copy fills one pair.
// Stage sizes: KC 32768 bytes, MC 33792; LDS holds A's two stages, then B's
// (at most 135168 bytes).
//
// Edge handling is that of gemm16_sched_kernel: each descriptor ends at its
// stored matrix's last element; a copy that must bring zeros has a per-lane
// offset past that end by itself (rows of a KC factor past the tile's edge
// in every phase; chunks or rows at k >= K in the last phase, whose copies
// take per-lane offsets with the phase folded in and a scalar offset of 0);
// the column overhang of an MC factor reads the next row (only C entries
// outside the matrix use it) or, in the last row, its dwords up to the end
// and zeros past it.  K need only be even: the one chunk per row of a KC
// factor that straddles K is copied whole, and its values past K are zeroed
// in the last phase's fragments.
//
// The k order inside each instruction (k = 32 s + 8 (l / 16) + e of lane l)
// does not depend on how a factor is stored, so the four op pairs give the
// same bits on explicitly transposed copies.
#include "mfma16_common.h"

namespace gemmf32 {

namespace {

template <int BT>
struct WideTileKC {
    static constexpr bool IS_KC = true;
    static constexpr int STAGE_BYTES = 128 * BT;
    static constexpr int COPIES = BT / 32;                // 1 KB copies per wave and phase
    static constexpr int READS = BT / 32;                 // LDS reads per step (one per fragment)
    static constexpr int BASES = 2;                       // read bases (one per step)
    __host__ __device__ static constexpr int swz(int r) { return (r >> 1) & 7; }
    // Copy j (0 .. COPIES - 1) of wave w fills stage bytes 1024 q .. + 1023,
    // q = w + 4 j: rows 8 q .. + 7; lane l fills physical chunk l % 8 of row
    // 8 q + l / 8.
    __host__ __device__ static int copy_q(int w, int j) { return w + 4 * j; }
    __host__ __device__ static int copy_dst(int w, int j) { return 1024 * copy_q(w, j); }
    __host__ __device__ static int copy_row(int w, int j, int lane) { return 8 * copy_q(w, j) + lane / 8; }
    // k of lane l's 8 values relative to the phase, and their row (mn) in
    // the tile.
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        return 8 * ((lane % 8) ^ swz(copy_row(w, j, lane)));
    }
    __host__ __device__ static int copy_mn(int w, int j, int lane) { return copy_row(w, j, lane); }
    // Byte offset of those values from the stored matrix's base at k = 0.
    __host__ __device__ static int64_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        return 2 * ((int64_t)(mn0 + copy_row(w, j, lane)) * ld + copy_k(w, j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return 2 * (int64_t)k0; }
    // Lane l's read base (bytes from the stage) for step s and the wave's
    // span at mn (a multiple of 16): row mn + l % 16, logical chunk
    // 4 s + l / 16 (the swizzle depends on l % 16 only); fragment f, read h,
    // is at + read_imm(s, f, h).
    __host__ __device__ static uint32_t read_base(int lane, int mn, int s) {
        return (uint32_t)(128 * (mn + lane % 16) + 16 * ((4 * s + lane / 16) ^ swz(lane % 16)));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int s, int f, int h) { return 2048u * f + 0u * (s + h); }
};

template <int BT>
struct WideTileMC {
    static constexpr bool IS_KC = false;
    static constexpr int STAGE_BYTES = 32 * 1056;
    static constexpr int COPIES = 8;                      // 1 KB copies per wave and phase
    static constexpr int READS = BT / 16;                 // LDS reads per step (two per fragment)
    static constexpr int BASES = 1;
    // Pair and row in the pair of the phase's k row kappa.
    __host__ __device__ static constexpr int pair(int kappa) {
        return (kappa & 3) + 4 * ((kappa >> 3) & 3) + 16 * (kappa >> 5);
    }
    __host__ __device__ static constexpr int half(int kappa) { return (kappa >> 2) & 1; }
    // Copy j (0..7) of wave w fills pair q = w + 4 j; lane l brings row
    // l / 32 of the pair, values 8 (l % 32) .. + 7 (a 512-byte row slot; with
    // a tile of 192 values the lanes of values 192 .. 255 copy zeros).
    __host__ __device__ static int copy_q(int w, int j) { return w + 4 * j; }
    __host__ __device__ static int copy_dst(int w, int j) { return 1056 * copy_q(w, j); }
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        const int q = copy_q(w, j);
        return 32 * (q >> 4) + 8 * ((q >> 2) & 3) + 4 * (lane / 32) + (q & 3);
    }
    __host__ __device__ static int copy_mn(int w, int j, int lane) { return 8 * (lane % 32); }
    __host__ __device__ static int64_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        return 2 * ((int64_t)copy_k(w, j, lane) * ld + mn0 + copy_mn(w, j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return 2 * (int64_t)k0 * ld; }
    // Lane l (group g = l / 16, j = l % 16) addresses k row 8 g + j / 4 (pair
    // j / 4 + 4 g, row 0) of step 0, values mn + 4 (j % 4) .. + 3 (see
    // read_tr16): it then receives value mn + j, k rows 8 g .. + 3.  Step s
    // adds 16 pairs, read h a row (k + 4), fragment f 16 values.
    __host__ __device__ static uint32_t read_base(int lane, int mn, int /*s*/) {
        const int j = lane % 16, g = lane / 16;
        return (uint32_t)(1056 * (j / 4 + 4 * g) + 2 * (mn + 4 * (j % 4)));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int s, int f, int h) {
        return 16896u * s + 32u * f + 512u * h;
    }
};

template <bool KC, int BT>
using WideTile = std::conditional_t<KC, WideTileKC<BT>, WideTileMC<BT>>;

// Waits until at most N copies of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_copies_below() {
    static_assert(N == 10 || N == 12 || N == 13 || N == 14 || N == 16, "copy count");
    if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    if constexpr (N == 13) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
    if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

// BT: the tile's extent in M and N (256, or 192 or 160 for problems whose
// 256 x 256 tiles fill the CUs' rounds badly); each wave holds a quarter of
// it.
template <int FMT, bool KCA, bool KCB, int BT = 256>
__global__ __launch_bounds__(256)
void gemm16_wide_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    static_assert(BT == 256 || BT == 192 || BT == 160, "tile");
    constexpr int BM = BT, BN = BT, WM = BT / 2, WN = BT / 2, BK = 64, FM = BT / 32, FN = BT / 32;
    using TA = WideTile<KCA, BT>;
    using TB = WideTile<KCB, BT>;
    constexpr int SA = TA::STAGE_BYTES, SB = TB::STAGE_BYTES;
    constexpr int A_COPIES = TA::COPIES, NCOPY = TA::COPIES + TB::COPIES;   // per wave and phase
    constexpr int NMFMA = FM * FN;                        // matrix instructions per step
    constexpr int NREAD = TA::READS + TB::READS;          // LDS reads per step
    // One read after each of the first NREAD matrix instructions of a step:
    // within its first two thirds, or four fifths for the 25 instructions of
    // a 160 tile with both factors mn-contiguous (20 reads).
    static_assert(NREAD <= (BT == 160 ? 4 * NMFMA / 5 : 2 * NMFMA / 3), "reads within the step");
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * (SA + SB)];

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

    // Copies 0 .. A_COPIES - 1 fill A's tile, the rest B's (byte offsets: the
    // launcher keeps both operands below 2^31 bytes with a tile's overhang, so
    // a past-the-end offset plus any phase's scalar offset stays below 2^32).
    // Lanes of an mn-contiguous factor's copies beyond a narrower tile copy
    // zeros into unread bytes: their offsets lie past the end in every phase.
    constexpr uint32_t kPastEnd = 0x80000000u;              // beyond any descriptor here
    constexpr int CMAX = TA::COPIES > TB::COPIES ? TA::COPIES : TB::COPIES;
    constexpr bool DEAD_A = !KCA && BT < 256, DEAD_B = !KCB && BT < 256;   // such lanes exist
    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < CMAX; ++j) {
        if (j < TA::COPIES) doff[j] = (uint32_t)TA::copy_src(wave_u, j, lane, m0, p.lda);
        if (j < TB::COPIES) doff[A_COPIES + j] = (uint32_t)TB::copy_src(wave_u, j, lane, n0, p.ldb);
        if constexpr (DEAD_A)
            if (j < TA::COPIES && TA::copy_mn(wave_u, j, lane) >= BT) doff[j] = kPastEnd;
        if constexpr (DEAD_B)
            if (j < TB::COPIES && TB::copy_mn(wave_u, j, lane) >= BT) doff[A_COPIES + j] = kPastEnd;
    }
    constexpr int kRawBufferWord3 = 0x00020000;
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.A), (short)0, (int)(2 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.B), (short)0, (int)(2 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    const int P = ceil_div(p.K, BK);
    const int klast = (P - 1) * BK;                         // the last phase's first k
    uint32_t dlast[NCOPY];
#pragma unroll
    for (int j = 0; j < CMAX; ++j) {
        const int ka = klast + TA::copy_k(wave_u, j, lane);
        const int kb = klast + TB::copy_k(wave_u, j, lane);
        if (j < TA::COPIES)
            dlast[j] = ka >= p.K || (DEAD_A && doff[j] == kPastEnd) ? kPastEnd
                                                                     : doff[j] + (uint32_t)TA::phase_bytes(klast, p.lda);
        if (j < TB::COPIES)
            dlast[A_COPIES + j] = kb >= p.K || (DEAD_B && doff[A_COPIES + j] == kPastEnd)
                                      ? kPastEnd
                                      : doff[A_COPIES + j] + (uint32_t)TB::phase_bytes(klast, p.ldb);
    }
    // Copy j of the phase at k0 into stage buf; LAST: the phase is the last
    // (its offsets hold the phase; k0 is not used).
    auto copy = [&](int j, int k0, int buf, auto lastc) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(lastc)::value;
        const uint32_t voff = LAST ? dlast[j] : doff[j];
        if (j < A_COPIES) {
            const int soff = LAST ? 0 : (int)TA::phase_bytes(k0, p.lda);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(lds + buf * SA + TA::copy_dst(wave_u, j)), 16,
                (int)voff, soff, 0, 0);
        } else {
            const int soff = LAST ? 0 : (int)TB::phase_bytes(k0, p.ldb);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(lds + 2 * SA + buf * SB + TB::copy_dst(wave_u, j - A_COPIES)),
                16, (int)voff, soff, 0, 0);
        }
    };

    // Read bases (stage 0): one per step for a KC factor, one for an MC
    // factor; fragment, read (and an MC factor's step) are instruction
    // offsets, and a phase moves the bases to the other stage.
    uint32_t abase[TA::BASES], bbase[TB::BASES];
#pragma unroll
    for (int x = 0; x < TA::BASES; ++x) abase[x] = lds_addr(lds) + TA::read_base(lane, wm * WM, x);
#pragma unroll
    for (int x = 0; x < TB::BASES; ++x) bbase[x] = lds_addr(lds) + 2u * SA + TB::read_base(lane, wn * WN, x);

    // Fragments, two sets: a KC factor's as 128-bit values (one read each),
    // an MC factor's as the two 64-bit halves its two reads bring, put
    // together only as the matrix instruction's operand (held as 128-bit
    // values, the register allocator moved the accumulators around every
    // trip of the loop).
    u32x4 aq[2][FM], bq[2][FN];
    u32x2 ah[2][FM][2], bh[2][FN][2];
    static_assert(FM == FN, "square tiles");
    // Read i (0 .. READS - 1) of one factor's fragments of step s into set
    // (q, h): KC, fragment i; MC, half i % 2 of fragment i / 2.
    auto read_one = [&](auto tile, u32x4 (&q)[FM], u32x2 (&hv)[FM][2], const uint32_t* base, int s, int i)
                        __attribute__((always_inline)) {
        using T = decltype(tile);
        if constexpr (T::IS_KC) q[i] = lds_read128(base[s] + T::read_imm(s, i, 0));
        else hv[i / 2][i % 2] = read_tr16_off(base[0], (int)T::read_imm(s, i / 2, i % 2));
    };
    // Read i of step s into set t from the stage the bases point at: A's
    // reads first, then B's.
    auto read_op = [&](int s, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, aq[t], ah[t], abase, s, i);
        else read_one(TB{}, bq[t], bh[t], bbase, s, i - TA::READS);
    };
    auto frag_a = [&](int t, int i) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCA) return aq[t][i];
        else return u32x4{ah[t][i][0][0], ah[t][i][0][1], ah[t][i][1][0], ah[t][i][1][1]};
    };
    auto frag_b = [&](int t, int j) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCB) return bq[t][j];
        else return u32x4{bh[t][j][0][0], bh[t][j][0][1], bh[t][j][1][0], bh[t][j][1][1]};
    };
    auto flip_stage = [&](int cur) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < TA::BASES; ++x) abase[x] += cur ? (uint32_t)-SA : (uint32_t)SA;
#pragma unroll
        for (int x = 0; x < TB::BASES; ++x) bbase[x] += cur ? (uint32_t)-SB : (uint32_t)SB;
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        if constexpr (KCA) wait_tied(aq[t]);
        else wait_tied(ah[t]);
        if constexpr (KCB) wait_tied(bq[t]);
        else wait_tied(bh[t]);
    };
    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One step: the NMFMA matrix instructions on set t (block (q / FN, q %
    // FN) for instruction q); after instruction q, read q of step rs into set
    // t ^ 1 (if R and q < NREAD) and, if C, copy c of the phase at k_copy
    // into stage cbuf (the last phase if lastc) after instruction
    // NMFMA (c + 1) / NCOPY - 1 (every fourth for a 256 tile).
    auto step = [&](int t, auto reads, int rs, auto copies, int k_copy, int cbuf, auto lastc)
                    __attribute__((always_inline)) {
        constexpr bool R = decltype(reads)::value;
        constexpr bool C = decltype(copies)::value;
        unroll<NMFMA>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            constexpr int c = (NCOPY * (q + 1) - 1) / NMFMA;   // the copy that ends at q, if any
            acc[q / FN][q % FN] = mfma16x16<FMT>(frag_a(t, q / FN), frag_b(t, q % FN), acc[q / FN][q % FN]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (R && q < NREAD) {
                read_op(rs, t ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (C && NMFMA * (c + 1) / NCOPY - 1 == q) {
                copy(c, k_copy, cbuf, lastc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
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
    // Phase ph (stage ph & 1) between the barriers that end phases ph - 1 and
    // ph: step 0 (set 0; reads step 1 into set 1), the barrier (the copies
    // of phase ph + 1 have landed, the stage of phase ph is free), then step
    // 1 (set 1; reads step 0 of phase ph + 1 into set 0 and, if C, copies
    // phase ph + 2 into the freed stage, the last phase if lastc).
    auto phase = [&](int ph, auto copies, auto lastc) __attribute__((always_inline)) {
        const int cur = ph & 1;
        wait_set(0);
        step(0, yes{}, 1, no{}, 0, 0, no{});
        wait_set(1);
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(1, yes{}, 0, copies, (ph + 2) * BK, cur, lastc);
    };

    // Prologue: phases 0 and 1 in flight together; the first barrier waits
    // for phase 0 only (loads complete in order).  The copies of phase P - 1
    // take the last phase's offsets: here when P <= 2, else in the loop's
    // final pass (peeled).
    if (P == 1) {
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy(j, 0, 0, yes{});
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy(j, 0, 0, no{});
        if (P == 2) {
#pragma unroll
            for (int j = 0; j < NCOPY; ++j) copy(j, BK, 1, yes{});
        } else {
#pragma unroll
            for (int j = 0; j < NCOPY; ++j) copy(j, BK, 1, no{});
        }
        wait_copies_below<NCOPY>();
    }
    __syncthreads();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(0, 0, i);
    __builtin_amdgcn_sched_barrier(0);
    int ph = 0;
    for (; ph + 3 < P; ++ph) phase(ph, yes{}, no{});
    if (ph + 2 < P) {                                       // copies of the last phase
        phase(ph, yes{}, yes{});
        ++ph;
    }
    if (ph + 1 < P) {
        phase(ph, no{}, no{});
        ++ph;
    }
    // The last phase.  With K not a multiple of 8, the 16-byte chunk of a
    // k-contiguous factor that holds k = K - 1 also holds values past K (the
    // row's next elements, or padding); lane l's fragments of step s hold
    // k = klast + 32 s + 8 (l / 16) + e, e = 0..7, and those at k >= K are
    // set to zero here, so that they meet zeros of the other factor (its
    // rows at k >= K copied as zeros, or its own fragments so masked).
    auto mask_last = [&](int t, int s) __attribute__((always_inline)) {
        if constexpr (KCA || KCB) {
            const int kv = p.K - klast - 32 * s - 8 * (lane >> 4);   // values of the chunk below K
            u32x4 m;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                m[d] = (2 * d < kv ? 0x0000FFFFu : 0u) | (2 * d + 1 < kv ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                if constexpr (KCA) aq[t][f] &= m;
                if constexpr (KCB) bq[t][f] &= m;
            }
        }
    };
    wait_set(0);
    mask_last(0, 0);
    step(0, yes{}, 1, no{}, 0, 0, no{});
    wait_set(1);
    mask_last(1, 1);
    step(1, no{}, 0, no{}, 0, 0, no{});

    // Guarded store (edge tiles run whole and store only what lies inside
    // C): register r of block (i, j) of lane l is row 16 i + 4 (l / 16) + r,
    // column 16 j + l % 16 of the wave's span.  Consecutive stores cover one
    // row across the blocks (512 contiguous bytes per lane group for a 256
    // tile; measured 1 % faster at 8192^3 than block by block).
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

template <int FMT, bool KCA, bool KCB, int BT>
hipError_t launch_wide_kernel(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                              unsigned blocks) {
    hipLaunchKernelGGL((gemm16_wide_kernel<FMT, KCA, KCB, BT>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

template <int BT>
hipError_t launch_wide_tiles(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m) {
    const int tiles_m = ceil_div(p.M, BT), tiles_n = ceil_div(p.N, BT);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned nb = (unsigned)blocks;
    switch (4 * (format ? 1 : 0) + 2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_wide_kernel<0, true, false, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 1: return launch_wide_kernel<0, true, true, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 2: return launch_wide_kernel<0, false, false, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 3: return launch_wide_kernel<0, false, true, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 4: return launch_wide_kernel<1, true, false, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 5: return launch_wide_kernel<1, true, true, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        case 6: return launch_wide_kernel<1, false, false, BT>(p, s, tiles_m, tiles_n, group_m, nb);
        default: return launch_wide_kernel<1, false, true, BT>(p, s, tiles_m, tiles_n, group_m, nb);
    }
}

}  // namespace

// K even and > 0 (the last phase's values past K are masked), an
// mn-contiguous factor's width (M for A stored transposed, N for B as
// stored) even, 4-byte aligned bases, even leading dimensions, and stored
// factors below 2^31 bytes with a tile's overhang.  Every descriptor then
// ends on a dword boundary: the range check is per dword, so with K odd the
// last row's last value would share a dword with the bytes past the end and
// read as zero.
bool wide_fits(const Gemm16Args& p, int op_a, int op_b) {
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const bool widths = (op_a == 0 || p.M % 2 == 0) && (op_b != 0 || p.N % 2 == 0);
    return vec && widths && p.K > 0 && p.K % 2 == 0 && p.M > 0 && p.N > 0 &&
           2 * (a_rows + 256) * p.lda < (1ll << 31) &&
           2 * (b_rows + 256) * p.ldb < (1ll << 31);
}

hipError_t launch_wide16(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m) {
    return launch_wide_tiles<256>(p, s, format, op_a, op_b, group_m);
}

hipError_t launch_wide16_192(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m) {
    return launch_wide_tiles<192>(p, s, format, op_a, op_b, group_m);
}

hipError_t launch_wide16_160(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m) {
    return launch_wide_tiles<160>(p, s, format, op_a, op_b, group_m);
}

}  // namespace gemmf32
