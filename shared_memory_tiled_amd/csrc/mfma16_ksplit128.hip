// mfma16_ksplit128.hip -- the mixed-precision product (bfloat16 or binary16
// factors, binary32 accumulation) for a few hundred output tiles of
// 128 x 128: one tile per block, its K split over the block's four waves.
//
// The one-volume PMPP notes run the fully connected layer as a matrix
// product on matrix units fed FP16 or BF16 and accumulating in FP32
// (deep-learning chapter, "FC Layer = GEMM", "Mixed Precision"); this is
// that product with the tiled structure of the pages' shared-memory chapter
// (tiles staged in LDS, ghost zeros past the matrix edges, a guarded store).
//
// A 2048^3 product has 64 tiles of 256 x 256 for 256 CUs, and 256 of
// 128 x 128: one round of one tile per CU.  Each of the block's four waves
// (one per SIMD) computes the whole 128 x 128 tile -- 8 x 8 blocks of
// 16 x 16 on v_mfma_f32_16x16x32, 256 accumulators -- over every fourth
// 32-deep phase (wave w: phases w, w + 4, ...) from two LDS stages of its
// own (16 KB each), which only that wave copies into and reads: no wave
// waits for another before the end, where the four partial tiles are added
// in wave order through LDS (deterministic; the same bits for every op
// pair).  A 128 x 128 tile needs 64 bytes of operands per clock at the
// matrix cores' full rate, about twice what a CU's L2 path brings, so the
// copies, not the instructions, set the pace.
//
// A phase is 64 matrix instructions (block (q / 8, q % 8) for instruction
// q, 1024 matrix-core clocks).  A wave runs its phases at positions: the
// last phase first, then (with an odd count) a position that copies zeros,
// then phases 0, 1, ..; at least two positions, an even number.  During
// position s it copies position s + 2 into the stage position s came from
// (16 copies of 1 KB, one after every odd instruction below 32), then, once
// the copies of position s + 1 have landed, reads position s + 1's fragments
// into its other register set (one read after each instruction from 24
// on).  The two phases that need per-lane copy offsets -- the last and the
// first -- sit at positions 0 to 2, copied in the prologue and by the first
// two positions (peeled); every later position runs one and the same body
// with one kind of copy, so the loop has no branch inside (a branch between
// phases keeps an unread register set live across it, and 256 accumulators
// leave no room for that).  Copies and reads aimed past the last position
// fill, and read, stages that nothing uses afterwards.

// Tiles (per stage, 128 mn x 32 k):
//   KC (k-contiguous factor: A as stored, B stored transposed): 128 rows of
//      32 k (64 bytes), the 16-byte chunk c (8 k) of row r at
//      c ^ (2 ((r / 8) mod 2)) (the 64 x 64 k-split kernel's rows); a 1 KB
//      copy fills 16 rows; fragment f is one 128-bit read of row
//      16 f + l % 16, chunk l / 16.
//   MC (mn-contiguous factor: B as stored, A stored transposed): 32 k rows
//      of 128 values (256 bytes) in eight groups of four, group Q at byte
//      1056 Q (32 bytes of padding a group); k row r = 8 g + 4 h + q (g =
//      0..3, h = 0..1, q = 0..3) is row 2 (g / 2) + h of group q + 4 (g mod
//      2).  A 1 KB copy fills one group; fragment f is two ds_read_b64_tr_b16
//      reads (h = 0, 1) of k rows 8 (l / 16) + 4 h + (l % 16) / 4.  The 32
//      lanes of one read cycle address 8 k rows in 8 different groups, each
//      shifted by 8 banks against the last (1056 = 33 x 32 bytes).
// Either way one read base per lane and factor serves every block, read and
// stage (instruction offsets).
//
// Edges as in the 64 x 64 k-split kernel: phases aligned to the end of K (K
// a multiple of 8), so only phase 0 reaches below k = 0; every copy that
// must bring zeros is past its descriptor's end by its per-lane offset
// alone (rows of a KC factor past the tile's edge, chunks of an MC factor
// wholly past its last column, lanes of phase 0 below k = 0, positions
// holding no phase); the wave's first and last phases take the phase in
// their per-lane offsets with a scalar offset of 0, so that a chunk of an
// MC factor's last row across its last column meets the descriptor's end by
// its own offset (the range check is per dword, and the width is even).
#include "mfma16_common.h"

namespace gemmf32 {

namespace {

template <bool KC>
struct KsplitTile128 {
    static constexpr int ELEMS = 128 * 32;               // per stage
    static constexpr int BYTES = KC ? 8192 : 8 * 1056;   // per stage
    static constexpr int READS = KC ? 8 : 16;            // LDS reads per phase (8 fragments)
    static constexpr bool IS_KC = KC;
    // Copy j (0..7), lane l: the stored row (KC: mn; MC: k) and the logical
    // chunk of 8 values it brings, into LDS byte copy_dst(j) + 16 l.
    __host__ __device__ static int copy_row(int j, int lane) {
        if constexpr (KC) return 16 * j + lane / 4;
        const int pos = lane / 16;
        return 8 * (2 * (pos >> 1) + (j >> 2)) + 4 * (pos & 1) + (j & 3);
    }
    __host__ __device__ static int copy_chunk(int j, int lane) {
        return KC ? (lane % 4) ^ (((copy_row(j, lane) >> 3) & 1) << 1) : lane % 16;
    }
    __host__ __device__ static constexpr int copy_dst(int j) { return KC ? 1024 * j : 1056 * j; }
    // k (relative to the phase) and first mn (relative to the tile) of the 8
    // values lane l of copy j brings.
    __host__ __device__ static int copy_k(int j, int lane) { return KC ? 8 * copy_chunk(j, lane) : copy_row(j, lane); }
    __host__ __device__ static int copy_mn(int j, int lane) { return KC ? copy_row(j, lane) : 8 * copy_chunk(j, lane); }
    // Byte offset of those 8 values from the stored matrix's base at k = 0.
    __host__ __device__ static int64_t copy_src(int j, int lane, int mn0, int64_t ld) {
        return KC ? 2 * ((int64_t)(mn0 + copy_row(j, lane)) * ld + copy_k(j, lane))
                  : 2 * ((int64_t)copy_row(j, lane) * ld + mn0 + copy_mn(j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return KC ? 2 * (int64_t)k0 : 2 * (int64_t)k0 * ld; }
    // Read base of lane l (bytes from stage 0 of this tile) and the
    // instruction offset of read i of block f (KC: i = 0; MC: i = 0, 1).
    //   KC: row 16 f + l % 16, chunk l / 16
    //   MC: k row 8 (l / 16) + 4 i + (l % 16) / 4, values 16 f + 4 (l % 4) .. + 3
    __host__ __device__ static uint32_t read_base(int lane) {
        const int j = lane & 15, g = lane >> 4;
        if constexpr (KC) return (uint32_t)(64 * j + 16 * (g ^ (((j >> 3) & 1) << 1)));
        return (uint32_t)(1056 * ((j >> 2) + 4 * (g & 1)) + 512 * (g >> 1) + 8 * (j & 3));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int f, int i) { return KC ? 1024u * f : 256u * i + 32u * f; }
};

template <int FMT, bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm16_ksplit128_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    using TA = KsplitTile128<KCA>;
    using TB = KsplitTile128<KCB>;
    constexpr int BK = 32;                               // k per phase
    constexpr int STAGE = TA::BYTES + TB::BYTES;         // bytes per stage (16 .. 16.5 KB)
    constexpr int WAVE_BYTES = 2 * STAGE;                // two stages per wave
    constexpr int PART_BYTES = 4 * 8 * 1024;             // a wave's outgoing partial blocks, per round
    static_assert(PART_BYTES <= WAVE_BYTES, "partials fit in the wave's stages");
    constexpr int NREAD = TA::READS + TB::READS;         // 16 .. 32
    constexpr int RO = 24;                               // instruction after which the first read goes
    static_assert(RO + NREAD <= 64, "a phase's reads fit in its instructions");
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * WAVE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * 128;
    const int n0 = (in_g / gm) * 128;

    // This wave's phases: local phase lp is phase 4 lp + w, at k0 = kof(lp).
    // It runs them at positions 0 .. P2 - 1: position 0 holds the last phase,
    // then (with an odd count, after a position that copies zeros) phases 0,
    // 1, .., P - 2; a wave with fewer than two phases runs two positions,
    // the missing ones copying zeros.  The phases that need per-lane offsets
    // -- the last and the first -- thus sit at positions 0 .. 2, copied in
    // the prologue and by the first two phases (peeled), and every copy in
    // the loop is the same.
    const int nph = ceil_div(p.K, BK);
    const int kbase = p.K - BK * nph;                    // -24 .. 0, a multiple of 8
    const int P = nph > w ? (nph - 1 - w) / 4 + 1 : 0;
    const int odd = P & 1;
    const int P2 = P + odd < 2 ? 2 : P + odd;
    auto kof = [&](int lp) __attribute__((always_inline)) { return kbase + BK * (4 * lp + w); };
    auto phase_at = [&](int s) __attribute__((always_inline)) { return s == 0 ? P - 1 : s - 1 - odd; };

    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    constexpr int kRawBufferWord3 = 0x00020000;
    constexpr uint32_t kPastEnd = 0x80000000u;           // beyond any descriptor here
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.A), (short)0, (int)(2 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.B), (short)0, (int)(2 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    // Copies 0..7 fill A's tile, 8..15 B's (byte offsets below 2^31: the
    // launcher checks the operands' extents).  Chunks of an MC factor wholly
    // past its last column point past the end in every phase.
    uint32_t doff[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        doff[j] = (uint32_t)TA::copy_src(j, lane, m0, p.lda);
        doff[8 + j] = (uint32_t)TB::copy_src(j, lane, n0, p.ldb);
        if (!KCA && m0 + TA::copy_mn(j, lane) >= a_cols) doff[j] = kPastEnd;
        if (!KCB && n0 + TB::copy_mn(j, lane) >= b_cols) doff[8 + j] = kPastEnd;
    }
    unsigned char* const wl = lds + w * WAVE_BYTES;
    auto copy_at = [&](int j, uint32_t voff, int soff, int stage) __attribute__((always_inline)) {
        if (j < 8) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + TA::copy_dst(j)), 16,
                (int)voff, soff, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + TA::BYTES + TB::copy_dst(j - 8)),
                16, (int)voff, soff, 0, 0);
        }
    };
    // Copy j of the phase at position s >= 4 (phase s - 1 - odd >= 2, the
    // phase in the scalar offset) into `stage`; positions from P2 on copy
    // into stages nothing reads afterwards.
    auto copy = [&](int j, int s, int stage) __attribute__((always_inline)) {
        const int k0 = kof(s - 1 - odd);
        copy_at(j, doff[j], (int)(j < 8 ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb)), stage);
    };
    // Copy j of the phase at position s with the phase in each lane's offset
    // (scalar offset 0) into `stage`: lanes below k = 0 or at k >= K, chunks
    // past an MC factor's last column, and positions holding no phase point
    // past the end.
    auto copy_folded = [&](int j, int s, int stage) __attribute__((always_inline)) {
        const int lp = phase_at(s);
        const int k0 = kof(lp);
        const int kl = j < 8 ? TA::copy_k(j, lane) : TB::copy_k(j - 8, lane);
        const int64_t pb = j < 8 ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb);
        const bool inside = lp >= 0 && lp < P && k0 + kl >= 0 && k0 + kl < p.K && doff[j] != kPastEnd;
        copy_at(j, inside ? (uint32_t)((int64_t)doff[j] + pb) : kPastEnd, 0, stage);
    };

    // Read bases (bytes, stage 0); block, read and stage are instruction offsets.
    const uint32_t abase = lds_addr(wl) + TA::read_base(lane);
    const uint32_t bbase = lds_addr(wl) + (uint32_t)TA::BYTES + TB::read_base(lane);

    // Fragments, two sets: a KC factor's as 128-bit values (one read each),
    // an MC factor's as the two 64-bit halves its two reads bring, put
    // together only as the matrix instruction's operand.
    u32x4 aq[2][8], bq[2][8];
    u32x2 ah[2][8][2], bh[2][8][2];
    // Read i (0 .. READS - 1) of one factor's fragments of the phase in stage
    // STG into set (q, h): KC, fragment i; MC, half i % 2 of fragment i / 2.
    auto read_one = [&](auto tile, u32x4 (&q)[8], u32x2 (&hv)[8][2], uint32_t base, auto stg, int i)
                        __attribute__((always_inline)) {
        using T = decltype(tile);
        constexpr uint32_t SOFF = (uint32_t)STAGE * decltype(stg)::value;
        if constexpr (T::IS_KC) q[i] = lds_read128(base + SOFF + T::read_imm(i, 0));
        else hv[i / 2][i % 2] = read_tr16_off(base, (int)(SOFF + T::read_imm(i / 2, i % 2)));
    };
    auto read_op = [&](auto stg, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, aq[t], ah[t], abase, stg, i);
        else read_one(TB{}, bq[t], bh[t], bbase, stg, i - TA::READS);
    };
    auto frag_a = [&](int t, int i) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCA) return aq[t][i];
        else return u32x4{ah[t][i][0][0], ah[t][i][0][1], ah[t][i][1][0], ah[t][i][1][1]};
    };
    auto frag_b = [&](int t, int j) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KCB) return bq[t][j];
        else return u32x4{bh[t][j][0][0], bh[t][j][0][1], bh[t][j][1][0], bh[t][j][1][1]};
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        if constexpr (KCA) wait_tied(aq[t]);
        else wait_tied(ah[t]);
        if constexpr (KCB) wait_tied(bq[t]);
        else wait_tied(bh[t]);
    };

    floatx4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The phase at position lp in stage U = lp % 2, its fragments in set U:
    // the 64 matrix instructions; after odd instruction q < 32, copy q / 2 of
    // position lp + 2 into stage U (FOLDED: with per-lane offsets); after
    // instruction RO - 1, wait until only this phase's 12 copies so far may
    // be in flight (those of position lp + 1 have landed, in order); after
    // instruction q >= RO, read q - RO of position lp + 1 from stage U ^ 1
    // into set U ^ 1.
    auto phase = [&](auto uc, int lp, auto foldc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        using NEXT = std::integral_constant<int, U ^ 1>;
        unroll<64>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            acc[q / 8][q % 8] = mfma16x16<FMT>(frag_a(U, q / 8), frag_b(U, q % 8), acc[q / 8][q % 8]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (q % 2 == 1 && q < 32) {
                if constexpr (decltype(foldc)::value) copy_folded(q / 2, lp + 2, U);
                else copy(q / 2, lp + 2, U);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q == RO - 1) {
                asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q >= RO && q < RO + NREAD) {
                read_op(NEXT{}, U ^ 1, q - RO);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        wait_set(U ^ 1);
    };
    using s0 = std::integral_constant<int, 0>;
    using s1 = std::integral_constant<int, 1>;

#pragma unroll
    for (int j = 0; j < 16; ++j) copy_folded(j, 0, 0);
#pragma unroll
    for (int j = 0; j < 16; ++j) copy_folded(j, 1, 1);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");                  // position 0 has landed
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(s0{}, 0, i);
    wait_set(0);
    __builtin_amdgcn_sched_barrier(0);
    phase(s0{}, 0, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    phase(s1{}, 1, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    for (int pos = 2; pos < P2; pos += 2) {
        phase(s0{}, pos, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        phase(s1{}, pos + 1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
    }
    // the copies aimed past the last position land in this wave's stages
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Partial tiles, in two rounds.  In round a, wave v adds block row
    // 4 a + v of the tile (16 rows) over the four waves, in wave order, and
    // stores it.  Each wave writes its four block rows of the round into its
    // own stages (no copy in flight and no read pending, and no other wave
    // reads them before the barrier), block row 4 a + v at float 2048 v, each
    // as 16 rows of 128 floats, row-major, the 16-float segments of row rho
    // XORed by 16 ((rho / 4) mod 2): register r of block (i, j) of lane l
    // (row 4 (l / 16) + r, column 16 j + l % 16) is one 32-bit write per
    // (j, r), conflict free at 32 lanes a cycle.  Wave v then reads, for
    // it = 0..7, row 2 it + l / 32, columns 4 (l % 32) .. + 3 of its block
    // row from each wave -- one 128-bit read, conflict free under the
    // measured grouping -- adds them and stores the four values with one
    // 128-bit store (32 lanes: 512 contiguous bytes of a row of C).  (Taking
    // the block rows in order keeps the allocator from moving accumulators
    // inside the phase loop.)
    // (rho / 4) mod 2 is (l / 16) mod 2 for a write and (it / 2) mod 2 for a
    // read, so two per-lane bases each serve every address (instruction
    // offsets): writes of even and of odd j; reads without and with the XOR.
    const int b16 = (lane >> 4) & 1;
    float* const wbase_even = reinterpret_cast<float*>(wl) + 512 * (lane >> 4) + (lane & 15) + 16 * b16;
    float* const wbase_odd = reinterpret_cast<float*>(wl) + 512 * (lane >> 4) + (lane & 15) - 16 * b16;
    const int colq = 4 * (lane & 31);
    const float* const rbase0 = reinterpret_cast<const float*>(lds) + 2048 * w + 128 * (lane >> 5) + colq;
    const float* const rbase1 = reinterpret_cast<const float*>(lds) + 2048 * w + 128 * (lane >> 5) + (colq ^ 16);
    unroll<2>([&](auto ac) __attribute__((always_inline)) {
        constexpr int a = decltype(ac)::value;
        if constexpr (a == 1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // round 0 is read
        unroll<4>([&](auto vc) __attribute__((always_inline)) {
            constexpr int v = decltype(vc)::value;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ((j & 1) ? wbase_odd : wbase_even)[2048 * v + 128 * r + 16 * j] = acc[4 * a + v][j][r];
        });
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int rho = 2 * it + (lane >> 5);
            const float* const rb = ((it >> 1) & 1) ? rbase1 : rbase0;
            floatx4 sum = *reinterpret_cast<const floatx4*>(rb + 256 * it);
#pragma unroll
            for (int u = 1; u < 4; ++u) sum += *reinterpret_cast<const floatx4*>(rb + (WAVE_BYTES / 4) * u + 256 * it);
            const int row = m0 + 16 * (4 * a + w) + rho, col = n0 + colq;
            if (row >= p.M) continue;
            float* const c = p.C + (int64_t)row * p.ldc + col;
            if (col + 3 < p.N && ((reinterpret_cast<uintptr_t>(c) & 15) == 0)) {
                *reinterpret_cast<floatx4*>(c) = sum;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < p.N) c[e] = sum[e];
            }
        }
    });
}

template <int FMT, bool KCA, bool KCB>
hipError_t launch_ksplit128_kernel(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                   unsigned blocks) {
    hipLaunchKernelGGL((gemm16_ksplit128_kernel<FMT, KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

}  // namespace

// K a multiple of 8, an mn-contiguous factor's width even, 4-byte aligned
// bases, even leading dimensions, and stored factors below 2^31 bytes with
// a tile's overhang (32-bit offsets).
bool ksplit128_fits(const Gemm16Args& p, int op_a, int op_b) {
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const bool widths = (op_a == 0 || p.M % 2 == 0) && (op_b != 0 || p.N % 2 == 0);
    return vec && widths && p.K % 8 == 0 && p.K > 0 && p.M > 0 && p.N > 0 &&
           2 * (a_rows + 128) * p.lda < (1ll << 31) && 2 * (b_rows + 128) * p.ldb < (1ll << 31);
}

// format: 0 bfloat16, 1 binary16; op_a / op_b: 1 if that factor is stored
// transposed.  128 x 128 tiles, tile-row groups of group_m.
hipError_t launch_ksplit128(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b, int group_m) {
    const int tiles_m = ceil_div(p.M, 128), tiles_n = ceil_div(p.N, 128);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned nb = (unsigned)blocks;
    switch (4 * (format ? 1 : 0) + 2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_ksplit128_kernel<0, true, false>(p, s, tiles_m, tiles_n, group_m, nb);
        case 1: return launch_ksplit128_kernel<0, true, true>(p, s, tiles_m, tiles_n, group_m, nb);
        case 2: return launch_ksplit128_kernel<0, false, false>(p, s, tiles_m, tiles_n, group_m, nb);
        case 3: return launch_ksplit128_kernel<0, false, true>(p, s, tiles_m, tiles_n, group_m, nb);
        case 4: return launch_ksplit128_kernel<1, true, false>(p, s, tiles_m, tiles_n, group_m, nb);
        case 5: return launch_ksplit128_kernel<1, true, true>(p, s, tiles_m, tiles_n, group_m, nb);
        case 6: return launch_ksplit128_kernel<1, false, false>(p, s, tiles_m, tiles_n, group_m, nb);
        default: return launch_ksplit128_kernel<1, false, true>(p, s, tiles_m, tiles_n, group_m, nb);
    }
}

}  // namespace gemmf32
