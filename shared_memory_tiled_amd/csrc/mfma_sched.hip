// mfma_sched.hip -- rung 3 on four waves with an explicit instruction order.
//
// The tiled product of the pages' shared-memory chapter (PMPP chapter 5
// notes, sections 5.4-5.5: per phase every thread of a block copies part of
// an A and a B tile into shared memory, a barrier, the multiply-adds from the
// tiles, a barrier, and a guarded store at the edges) on 256 x 256 (or 128 x
// 128) output tiles, 32 k values per phase (K a multiple of 4; a last
// phase past K copies zeros there), two LDS
// stages so the copies of the next phase overlap the math of the current
// one.  Further down, the same schedule on 64 x 64 tiles whose four waves
// each take every fourth phase of the whole tile (gemm_f32_ksplit_kernel,
// K a multiple of 4).
//
// Four waves in 2 x 2, each owning a 128 x 128 block of C as 4 x 4 blocks of
// 32 x 32 (v_mfma_f32_32x32x2_f32, 256 accumulator registers per lane).  A
// wave tile of 128 x 128 reads 256 values of LDS per k for 32768 products,
// against 192 for 16384 on the eight-wave 128 x 64 tiles of the other
// kernels: a third less LDS traffic per flop.  With one wave per SIMD no
// second wave covers a wait, so the kernel places every instruction itself:
// a step is the 64 matrix instructions of 8 k values; while one step's
// fragments feed the matrix core, the next step's are read from LDS (eight
// 128-bit reads after the first eight instructions) and every eighth
// instruction is followed by one 1 KB global -> LDS copy of the next phase.
// Copies 0..7 of a phase are issued in the last step of the phase before the
// previous one, after the barrier, and 8..15 in step 0 of the previous phase,
// so every copy has three steps to land before the barrier that ends that
// phase.
//
// LDS tiles (per stage, 32 KB each):
//   k-contiguous factor (A as stored, B stored transposed): 256 rows of 32
//     floats (128 bytes).  Chunk c (16 bytes) of row r sits at position
//     c ^ ((r / 2) mod 8): the 16 rows one 128-bit read cycle touches (two
//     per 64-bank sweep) land on 16 different 4-bank groups.  A copy fills 8
//     rows.  Lane l of a wave reads row 32 f + l % 32, k = kg + 4 (l / 32)
//     .. + 3 for block f: its four values of instruction s = 0..3.
//   mn-contiguous factor (B as stored, A stored transposed): 32 k rows of
//     256 floats (1 KB, one copy each), unpadded.  Lane l reads the 128-bit
//     run of columns 4 (l % 32) .. + 3 of k row kg + 4 (l / 32) + s: one
//     value for each of the wave's four blocks, so block f of this factor
//     covers the columns 4 c + f (c = 0..31) of the wave's 128-wide span.
//     Sixteen lanes of one read cycle cover 256 consecutive bytes: no bank
//     conflict, and four reads per step instead of sixteen 32-bit ones.
// A block's k order (instruction s of group kg takes k = kg + s and
// kg + 4 + s) is that of the eight-wave kernels, so both give the same bits.
#include "launch.h"

#include <type_traits>
#include <utility>

namespace gemmf32 {

namespace {

constexpr int kSBK = 32;                 // k values per phase

__host__ __device__ constexpr int sched_swz(int r) { return (r >> 1) & 7; }

template <typename F, int... Q>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Q...>) {
    (f(std::integral_constant<int, Q>{}), ...);
}
// f(std::integral_constant<int, q>{}) for q = 0 .. N - 1, in order, each q a
// compile-time constant (so the arrays it indexes stay in registers).
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// 16 and 8 bytes of LDS at a byte address.
__device__ __forceinline__ floatx4 lds_read128(uint32_t lds_byte_addr) {
    typedef const __attribute__((address_space(3))) floatx4 lds_floatx4;
    return *(lds_floatx4*)(uintptr_t)lds_byte_addr;
}
typedef float floatx2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ floatx2 lds_read64(uint32_t lds_byte_addr) {
    typedef const __attribute__((address_space(3))) floatx2 lds_floatx2;
    return *(lds_floatx2*)(uintptr_t)lds_byte_addr;
}

// Byte address inside LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Waits for all outstanding LDS reads; the fragments pass through the wait
// as operands, so no use of them is scheduled before it (and the compiler
// adds no wait of its own that would also cover reads issued later).
__device__ __forceinline__ void wait_tied(floatx4 (&x)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : : "memory");
}

// One factor's tile: MNT (256, 128 or 64) rows or columns of op(X) by 32 k
// per stage; each wave holds F (4, 2 or 1) blocks of 32 of it.  KC: stored
// k-contiguous.  Copy j of wave w: one of the 4 MNT / 32 copies of a stage,
// dealt to four waves in turn.
template <bool KC, int MNT, int F>
struct SchedTileF32 {
    static_assert((MNT == 256 || MNT == 128 || MNT == 64) && (F == 4 || F == 2 || F == 1), "tile shape");
    static constexpr int WORDS = MNT * kSBK;              // floats per stage
    static constexpr int COPIES = MNT / 32;               // 1 KB copies per wave and phase
    static constexpr int RPC = KC ? 8 : 256 / MNT;        // stored rows per copy
    static constexpr int READS = KC ? F : 4;              // LDS reads per step
    static constexpr bool IS_KC = KC;
    static constexpr int FV = F;
    // First float, inside the tile stage, that copy j of wave w fills.
    __host__ __device__ static int copy_dst(int w, int j) {
        return KC ? 8 * (w + 4 * j) * kSBK : RPC * (w + 4 * j) * MNT;
    }
    // Byte offset of lane l's 16 bytes of copy j from the stored matrix's
    // base at k = 0 (mn0: the tile's first row or column of op(X)).
    __host__ __device__ static uint32_t copy_src(int w, int j, int lane, int mn0, int64_t ld) {
        if constexpr (KC) {
            const int row = 8 * (w + 4 * j) + lane / 8;
            return 4u * (uint32_t)((mn0 + row) * ld + 4 * ((lane % 8) ^ sched_swz(row)));
        } else {
            constexpr int LPR = 64 / RPC;                   // lanes per stored row
            const int row = RPC * (w + 4 * j) + lane / LPR;
            return 4u * (uint32_t)(row * ld + mn0 + 4 * (lane % LPR));
        }
    }
    // mn-contiguous only: first column, relative to the tile's first one, of
    // lane l's 16 bytes (the same in every copy).
    __host__ __device__ static int copy_mn(int lane) { return 4 * (lane % (64 / RPC)); }
    // k of lane l's 16 bytes of copy j of wave w, relative to the phase's
    // first k.
    __host__ __device__ static int copy_k(int w, int j, int lane) {
        if constexpr (KC) {
            const int row = 8 * (w + 4 * j) + lane / 8;
            return 4 * ((lane % 8) ^ sched_swz(row));
        } else {
            return RPC * (w + 4 * j) + lane / (64 / RPC);
        }
    }
    // Byte offset of the phase at k0 from the phase at 0.
    __host__ __device__ static int phase_bytes(int k0, int64_t ld) { return KC ? 4 * k0 : 4 * k0 * (int)ld; }
    // LDS byte offset, inside stage 0 of this factor, of lane (li, lh)'s read
    // i of step s for the wave whose span of 32 F starts at mn:
    //   KC: block i's row mn + 32 i + li, logical chunk 2 s + lh (128 bits);
    //   MC: k row 8 s + 4 lh + i, columns mn + F li .. + F - 1 (F values).
    // Either way a per-lane base plus a compile-time part (4096 i for KC, as
    // the swizzle of row mn + 32 i + li depends on li only; 4 MNT (8 s + i)
    // for MC).
    __host__ __device__ static uint32_t read_base(int mn, int s, int li, int lh) {
        return KC ? 4u * (uint32_t)((mn + li) * kSBK + 4 * ((2 * s + lh) ^ sched_swz(li)))
                  : 4u * (uint32_t)(4 * lh * MNT + mn + F * li);
    }
    __host__ __device__ static constexpr uint32_t read_imm(int s, int i) {
        return KC ? 4096u * (uint32_t)i : 4u * MNT * (uint32_t)(8 * s + i);
    }
};

// Operand of block f for instruction e from a lane's four reads x: KC, value
// e of read f; MC, value f of read e.
template <bool KC>
__device__ __forceinline__ float operand(const floatx4 (&x)[4], int f, int e) {
    return KC ? x[f][e] : x[e][f];
}

// FM x FN blocks of 32 x 32 per wave, 2 x 2 waves: 256 x 256 tiles (FM =
// FN = 4) or 128 x 128 (FM = FN = 2).
template <int FM, int FN, bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm_f32_sched_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    constexpr int WM = 32 * FM, WN = 32 * FN, BM = 2 * WM, BN = 2 * WN;
    using TA = SchedTileF32<KCA, BM, FM>;
    using TB = SchedTileF32<KCB, BN, FN>;
    constexpr int A_COPIES = TA::COPIES, NCOPY = TA::COPIES + TB::COPIES, HALF = NCOPY / 2;
    constexpr int NREAD = TA::READS + TB::READS;
    constexpr int NMFMA = 4 * FM * FN;                    // matrix instructions per step
    constexpr int CSTRIDE = NMFMA / HALF;                 // a copy after every CSTRIDE-th of them
    static_assert(NCOPY % 2 == 0 && NREAD <= NMFMA && CSTRIDE >= 1, "schedule");
    constexpr int A_ST = TA::WORDS, B_ST = TB::WORDS;
    // A stage 0, A stage 1, B stage 0, B stage 1.
    __shared__ __attribute__((aligned(16))) float lds[2 * (A_ST + B_ST)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave_u / 2, wn = wave_u % 2;
    const int li = lane & 31, lh = lane >> 5;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    // Copies 0..7 fill A's tile, 8..15 B's (byte offsets: the launcher keeps
    // both stored matrices below 2^31 bytes).
    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        doff[j] = TA::copy_src(wave_u, j, lane, m0, p.lda);
        doff[A_COPIES + j] = TB::copy_src(wave_u, j, lane, n0, p.ldb);
    }
    constexpr int kRawBufferWord3 = 0x00020000;
    // Each descriptor ends exactly at its stored matrix's last element, and
    // every copy that must bring zeros gets them from a per-lane offset that
    // by itself lies at or past that end (the scalar offset, which holds the
    // phase, never decides it).  An edge tile's copies past the last row of
    // a k-contiguous factor have such offsets in every phase.  Past the last
    // column of an mn-contiguous factor they read the next row, which only
    // ever meets C entries outside the matrix, never stored; an
    // mn-contiguous factor's extent is a multiple of 4, so no 16-byte chunk
    // straddles an edge.  The last phase's copies take their own per-lane
    // offsets (dlast) with the phase folded in and a scalar offset of 0:
    // K is a multiple of 4, and its chunks or rows at k >= K are pointed
    // past the end (kPastEnd), so they copy zeros, as does the column
    // overhang of the last row; the other kernels' ghost phases hold the
    // same zeros, so all still give the same bits.
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.A), (short)0, (int)(4 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.B), (short)0, (int)(4 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    const int P = ceil_div(p.K, kSBK);
    constexpr uint32_t kPastEnd = 0x80000000u;              // beyond any descriptor here
    const int klast = (P - 1) * kSBK;                       // the last phase's first k
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
                rsrc_a, (__attribute__((address_space(3))) void*)(lds + buf * A_ST + TA::copy_dst(wave_u, j)), 16,
                (int)voff, soff, 0, 0);
        } else {
            const int soff = LAST ? 0 : TB::phase_bytes(k0, p.ldb);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(lds + 2 * A_ST + buf * B_ST + TB::copy_dst(wave_u, j - A_COPIES)),
                16, (int)voff, soff, 0, 0);
        }
    };

    // Per-lane read bases (stage 0): KC needs one per step, MC one in all.
    constexpr int SA = KCA ? 4 : 1, SB = KCB ? 4 : 1;
    uint32_t abase[SA], bbase[SB];
    const uint32_t lds0 = lds_addr(lds);
#pragma unroll
    for (int s = 0; s < SA; ++s) abase[s] = lds0 + TA::read_base(wm * WM, s, li, lh);
#pragma unroll
    for (int s = 0; s < SB; ++s) bbase[s] = lds0 + 8u * A_ST + TB::read_base(wn * WN, s, li, lh);

    floatx4 a[2][4], b[2][4];
    // Read i (0..7) of step s into set t, A's four first, from the stage the
    // bases point at: step and read index go into the instruction's offset
    // field.  The bases move to the other stage once per phase (flip_stage),
    // so the loop holds 2..8 vector ALU instructions per phase besides the
    // matrix ones, not one per read: each placed between two matrix
    // instructions was measured to cost the matrix core about 14 cycles
    // (scalar ones cost nothing).
    // An mn-contiguous read of F = 2 values fills the first two of each
    // fragment slot (the operand picks only those).
    auto read_one = [&](auto tile, floatx4 (&x)[4], uint32_t base, int s, int i) __attribute__((always_inline)) {
        using T = decltype(tile);
        const uint32_t addr = base + T::read_imm(s, i);
        if constexpr (T::IS_KC || T::FV == 4) {
            x[i] = lds_read128(addr);
        } else {
            const floatx2 v = lds_read64(addr);
            x[i][0] = v[0];
            x[i][1] = v[1];
        }
    };
    auto read_op = [&](int s, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, a[t], abase[KCA ? s : 0], s, i);
        else read_one(TB{}, b[t], bbase[KCB ? s : 0], s, i - TA::READS);
    };
    // Point the read bases at the other stage (from stage cur to cur ^ 1).
    auto flip_stage = [&](int cur) __attribute__((always_inline)) {
        const uint32_t da = cur ? (uint32_t)(-4 * A_ST) : (uint32_t)(4 * A_ST);
        const uint32_t db = cur ? (uint32_t)(-4 * B_ST) : (uint32_t)(4 * B_ST);
#pragma unroll
        for (int s = 0; s < SA; ++s) abase[s] += da;
#pragma unroll
        for (int s = 0; s < SB; ++s) bbase[s] += db;
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One step: the 4 FM FN matrix instructions on fragment set t
    // (instruction q: e = q / (FM FN), block (q / FN % FM, q % FN)); after the
    // q-th (q < NREAD), read q of step rs into set t ^ 1 (if R) and, after
    // every CSTRIDE-th, copy CB + q / CSTRIDE (while below CE) of the phase at
    // k_copy (the last phase if lastc) into stage cbuf.
    auto step = [&](int t, auto reads, int rs, auto cb, auto ce, int k_copy, int cbuf,
                    auto lastc) __attribute__((always_inline)) {
        constexpr bool R = decltype(reads)::value;
        constexpr int CB = decltype(cb)::value, CE = decltype(ce)::value;
        unroll<NMFMA>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            constexpr int e = q / (FM * FN), i = (q / FN) % FM, j = q % FN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(operand<KCA>(a[t], i, e),
                                                             operand<KCB>(b[t], j, e), acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (R && q < NREAD) {
                read_op(rs, t ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q % CSTRIDE == CSTRIDE - 1 && CB + q / CSTRIDE < CE) {
                copy(CB + q / CSTRIDE, k_copy, cbuf, lastc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
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
    using cH = std::integral_constant<int, HALF>;
    using cN = std::integral_constant<int, NCOPY>;
    // Steps 0..2 of the phase (step 0's fragments already read) and the wait
    // for step 3's; copies HALF.. of the phase at k_copy (the last phase if
    // lastc) into stage cbuf with step 0 if WC.
    auto steps012 = [&](auto wc, int k_copy, int cbuf, auto lastc) __attribute__((always_inline)) {
        constexpr bool WC = decltype(wc)::value;
        wait_set(0);
        if constexpr (WC) step(0, yes{}, 1, cH{}, cN{}, k_copy, cbuf, lastc);
        else step(0, yes{}, 1, c0{}, c0{}, 0, 0, no{});
        wait_set(1);
        step(1, yes{}, 2, c0{}, c0{}, 0, 0, no{});
        wait_set(0);
        step(0, yes{}, 3, c0{}, c0{}, 0, 0, no{});
        wait_set(1);
    };

    // Stage ph & 1 holds phase ph.  Between the barriers that end phases
    // ph - 1 and ph run the deferred last step of phase ph - 1 (with copies
    // 0..HALF-1 of phase ph + 1 and the first reads of phase ph, the read
    // bases already on its stage) and steps 0..2 of phase ph (the other
    // copies with step 0).  The copies of phase P - 1 take the last phase's
    // offsets: in the prologue when P <= 2, else in the loop's final pass
    // (peeled) and the block after it.
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
        for (int j = 0; j < HALF; ++j) copy(j, kSBK, 1, yes{});
    } else if (P > 2) {
#pragma unroll
        for (int j = 0; j < HALF; ++j) copy(j, kSBK, 1, no{});
    }
    __builtin_amdgcn_sched_barrier(0);
    int ph = 0;
    for (; ph + 3 < P; ++ph) {
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kSBK, cur ^ 1, no{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(1, yes{}, 0, c0{}, cH{}, (ph + 2) * kSBK, cur, no{});
    }
    if (ph + 2 < P) {                                       // copies 0..HALF-1 of the last phase
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kSBK, cur ^ 1, no{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(1, yes{}, 0, c0{}, cH{}, (ph + 2) * kSBK, cur, yes{});
        ++ph;
    }
    if (ph + 1 < P) {                                       // the rest of the last phase's copies
        const int cur = ph & 1;
        steps012(yes{}, (ph + 1) * kSBK, cur ^ 1, yes{});
        flip_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        step(1, yes{}, 0, c0{}, c0{}, 0, 0, no{});
        ++ph;
    }
    steps012(no{}, 0, 0, no{});
    step(1, no{}, 0, c0{}, c0{}, 0, 0, no{});

    // Guarded store.  Register r of lane (li, lh) is row rho = 8 (r / 4) +
    // 4 lh + r % 4 and column li of its 32 x 32 block; block (i, j) of a
    // k-contiguous A holds rows 32 i + rho of the wave's span, of an
    // mn-contiguous A rows FM rho + i; likewise for B's columns.  With B
    // mn-contiguous the FN blocks j of one row are FN adjacent columns: one
    // 128- or 64-bit store (N is a multiple of 4, so all are in or out).
    const int col0 = n0 + wn * WN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rho = 8 * (r >> 2) + 4 * lh + (r & 3);
            const int row = m0 + wm * WM + (KCA ? 32 * i + rho : FM * rho + i);
            if (row >= p.M) continue;
            float* crow = p.C + (int64_t)row * p.ldc + col0;
            if constexpr (!KCB) {
                if (col0 + FN * li < p.N) {
                    if constexpr (FN == 4) {
                        const floatx4 v = {acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]};
                        *reinterpret_cast<floatx4*>(crow + 4 * li) = v;
                    } else {
                        const floatx2 v = {acc[i][0][r], acc[i][1][r]};
                        *reinterpret_cast<floatx2*>(crow + 2 * li) = v;
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    if (col0 + 32 * j + li < p.N) crow[32 * j + li] = acc[i][j][r];
            }
        }
}

// Small products: 64 x 64 tiles, one per workgroup, whose four waves each
// compute the whole tile over every fourth phase (wave w: phases w, w + 4,
// ...) from two LDS stages of their own, which only that wave copies into
// and reads.  The waves never wait for each other before the end, where
// their four partial tiles meet in LDS and are added in wave order (so the
// result is deterministic; its rounding differs from the one-wave-per-block
// kernels, within the same bound).  Per wave the schedule above on a 64 x
// 64 wave tile (2 x 2 blocks): 16 matrix instructions per step, the 16 1 KB
// copies of a phase after every second of them in two steps, and one wait
// for the wave's own copies where the kernel above has its barrier.
//
// K need only be a multiple of 4: the phases are aligned to the end of K,
// phase g covering k = K - 32 (P - g) .. + 31 for P = ceil(K / 32) phases,
// so only phase 0 can reach below k = 0, and its lanes there are pointed
// past the end of their descriptor and copy zeros.
//
// TL (a measurement build, never the product's): every wave of the first
// timeline_blocks blocks also records, at words 8 (4 b + w) .. + 7 of
// `timeline`, the 100 MHz real-time counter at its start, when its first
// phase has landed, after its last matrix instruction is issued, after the
// barrier before the partial tiles are added, and once its stores have
// completed; then its shader-clock cycles between the first and the last,
// its phase count and its block.
template <bool KCA, bool KCB, bool TL = false>
__global__ __launch_bounds__(256)
void gemm_f32_ksplit_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m, uint32_t* timeline,
                            int timeline_blocks) {
    constexpr int FM = 2, FN = 2, BM = 64, BN = 64;
    using TA = SchedTileF32<KCA, BM, FM>;
    using TB = SchedTileF32<KCB, BN, FN>;
    constexpr int A_COPIES = 4 * TA::COPIES, NCOPY = A_COPIES + 4 * TB::COPIES, HALF = NCOPY / 2;
    constexpr int NREAD = TA::READS + TB::READS;
    constexpr int NMFMA = 4 * FM * FN;
    constexpr int CSTRIDE = NMFMA / HALF;
    static_assert(NCOPY == 16 && NREAD <= NMFMA && CSTRIDE == 2, "schedule");
    constexpr int A_ST = TA::WORDS, B_ST = TB::WORDS;
    constexpr int WAVE_WORDS = 2 * (A_ST + B_ST);            // A stage 0, 1, B stage 0, 1
    constexpr int PART_WORDS = FM * FN * 16 * 64;            // one wave's partial tile
    static_assert(PART_WORDS <= WAVE_WORDS, "partials reuse the stages");
    __shared__ __attribute__((aligned(16))) float lds[4 * WAVE_WORDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    uint32_t tl[5] = {};
    uint32_t tl_cycles = 0;
    auto mark = [&](int i) __attribute__((always_inline)) {
        if constexpr (TL) {
            __builtin_amdgcn_sched_barrier(0);
            tl[i] = (uint32_t)__builtin_amdgcn_s_memrealtime();
            if (i == 0) {                     // a wave without phases: empty phase loop
                tl_cycles = (uint32_t)__builtin_amdgcn_s_memtime();
                tl[1] = tl[2] = tl[0];
            }
            if (i == 4) tl_cycles = (uint32_t)__builtin_amdgcn_s_memtime() - tl_cycles;
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    mark(0);

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    // This wave's phases: local phase lp is phase 4 lp + w, at k0 = kof(lp).
    const int nph = ceil_div(p.K, kSBK);
    const int kbase = p.K - kSBK * nph;                      // -31 .. 0
    const int P = nph > w ? (nph - 1 - w) / 4 + 1 : 0;
    auto kof = [&](int lp) __attribute__((always_inline)) { return kbase + kSBK * (4 * lp + w); };

    // Descriptors end exactly at each stored matrix's last element, and a
    // copy that must bring zeros gets them from a per-lane offset that by
    // itself lies at or past that end (never from the scalar offset, which
    // holds the phase): rows of a k-contiguous factor past the tile's edge
    // have such offsets; the 16-byte chunks of an mn-contiguous factor past
    // its last column (which would only meet C entries outside the matrix;
    // its extent is a multiple of 4, so a chunk is wholly in or out) are
    // pointed past the end (kPastEnd) in every phase; and phase 0's lanes
    // below k = 0 are pointed there too (copy_first).  Every other lane
    // addresses an element of the matrix in every phase.
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    constexpr int kRawBufferWord3 = 0x00020000;
    constexpr uint32_t kPastEnd = 0x80000000u;               // beyond any descriptor here
    // Copy j < 8 fills A's tile, j >= 8 B's; within a factor copy j is copy
    // j / 4 of "wave" j % 4 of the shared layout, so one wave covers it all.
    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        doff[j] = TA::copy_src(j % 4, j / 4, lane, m0, p.lda);
        doff[A_COPIES + j] = TB::copy_src(j % 4, j / 4, lane, n0, p.ldb);
        if (!KCA && m0 + TA::copy_mn(lane) >= a_cols) doff[j] = kPastEnd;
        if (!KCB && n0 + TB::copy_mn(lane) >= b_cols) doff[A_COPIES + j] = kPastEnd;
    }
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.A), (short)0, (int)(4 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.B), (short)0, (int)(4 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    float* const wl = lds + w * WAVE_WORDS;
    auto copy_at = [&](int j, uint32_t voff, int soff, int buf) __attribute__((always_inline)) {
        if (j < A_COPIES) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(wl + buf * A_ST + TA::copy_dst(j % 4, j / 4)),
                16, (int)voff, soff, 0, 0);
        } else {
            const int jb = j - A_COPIES;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(wl + 2 * A_ST + buf * B_ST + TB::copy_dst(jb % 4, jb / 4)),
                16, (int)voff, soff, 0, 0);
        }
    };
    auto copy = [&](int j, int k0, int buf) __attribute__((always_inline)) {
        copy_at(j, doff[j], j < A_COPIES ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb), buf);
    };
    // The wave's first phase (k0 <= 0 only for phase 0), into stage 0: the
    // phase offset goes into each lane's offset, and lanes whose k is
    // negative point past the end.
    auto copy_first = [&]() __attribute__((always_inline)) {
        const int k0 = kof(0);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) {
            const bool is_a = j < A_COPIES;
            const int jj = is_a ? j : j - A_COPIES;
            const int kl = is_a ? TA::copy_k(jj % 4, jj / 4, lane) : TB::copy_k(jj % 4, jj / 4, lane);
            const int pb = is_a ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb);
            copy_at(j, k0 + kl >= 0 && doff[j] != kPastEnd ? doff[j] + (uint32_t)pb : kPastEnd, 0, 0);
        }
    };

    constexpr int SA = KCA ? 4 : 1, SB = KCB ? 4 : 1;
    uint32_t abase[SA], bbase[SB];
    const uint32_t wl0 = lds_addr(wl);
#pragma unroll
    for (int s = 0; s < SA; ++s) abase[s] = wl0 + TA::read_base(0, s, li, lh);
#pragma unroll
    for (int s = 0; s < SB; ++s) bbase[s] = wl0 + 8u * A_ST + TB::read_base(0, s, li, lh);

    floatx4 a[2][4], b[2][4];
    auto read_one = [&](auto tile, floatx4 (&x)[4], uint32_t base, int s, int i) __attribute__((always_inline)) {
        using T = decltype(tile);
        const uint32_t addr = base + T::read_imm(s, i);
        if constexpr (T::IS_KC) {
            x[i] = lds_read128(addr);
        } else {
            const floatx2 v = lds_read64(addr);
            x[i][0] = v[0];
            x[i][1] = v[1];
        }
    };
    auto read_op = [&](int s, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, a[t], abase[KCA ? s : 0], s, i);
        else read_one(TB{}, b[t], bbase[KCB ? s : 0], s, i - TA::READS);
    };
    auto flip_stage = [&](int cur) __attribute__((always_inline)) {
        const uint32_t da = cur ? (uint32_t)(-4 * A_ST) : (uint32_t)(4 * A_ST);
        const uint32_t db = cur ? (uint32_t)(-4 * B_ST) : (uint32_t)(4 * B_ST);
#pragma unroll
        for (int s = 0; s < SA; ++s) abase[s] += da;
#pragma unroll
        for (int s = 0; s < SB; ++s) bbase[s] += db;
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto step = [&](int t, auto reads, int rs, auto cb, auto ce, int k_copy,
                    int cbuf) __attribute__((always_inline)) {
        constexpr bool R = decltype(reads)::value;
        constexpr int CB = decltype(cb)::value, CE = decltype(ce)::value;
        unroll<NMFMA>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            constexpr int e = q / (FM * FN), i = (q / FN) % FM, j = q % FN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(operand<KCA>(a[t], i, e),
                                                             operand<KCB>(b[t], j, e), acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (R && q < NREAD) {
                read_op(rs, t ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (q % CSTRIDE == CSTRIDE - 1 && CB + q / CSTRIDE < CE) {
                copy(CB + q / CSTRIDE, k_copy, cbuf);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        wait_tied(a[t]);
        wait_tied(b[t]);
    };
    // This wave's copies have landed (no other wave reads its stages).
    auto wait_copies = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    using yes = std::true_type;
    using no = std::false_type;
    using c0 = std::integral_constant<int, 0>;
    using cH = std::integral_constant<int, HALF>;
    using cN = std::integral_constant<int, NCOPY>;
    auto steps012 = [&](auto wc, int k_copy, int cbuf) __attribute__((always_inline)) {
        constexpr bool WC = decltype(wc)::value;
        wait_set(0);
        if constexpr (WC) step(0, yes{}, 1, cH{}, cN{}, k_copy, cbuf);
        else step(0, yes{}, 1, c0{}, c0{}, 0, 0);
        wait_set(1);
        step(1, yes{}, 2, c0{}, c0{}, 0, 0);
        wait_set(0);
        step(0, yes{}, 3, c0{}, c0{}, 0, 0);
        wait_set(1);
    };

    // Stage lp & 1 holds local phase lp; the order of the kernel above.
    if (P > 0) {
        copy_first();
        wait_copies();
        mark(1);
#pragma unroll
        for (int i = 0; i < NREAD; ++i) read_op(0, 0, i);
        if (P > 1) {
#pragma unroll
            for (int j = 0; j < HALF; ++j) copy(j, kof(1), 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        int lp = 0;
        for (; lp + 2 < P; ++lp) {
            const int cur = lp & 1;
            steps012(yes{}, kof(lp + 1), cur ^ 1);
            flip_stage(cur);
            __builtin_amdgcn_sched_barrier(0);
            wait_copies();
            step(1, yes{}, 0, c0{}, cH{}, kof(lp + 2), cur);
        }
        if (lp + 1 < P) {
            const int cur = lp & 1;
            steps012(yes{}, kof(lp + 1), cur ^ 1);
            flip_stage(cur);
            __builtin_amdgcn_sched_barrier(0);
            wait_copies();
            step(1, yes{}, 0, c0{}, c0{}, 0, 0);
        }
        steps012(no{}, 0, 0);
        step(1, no{}, 0, c0{}, c0{}, 0, 0);
        mark(2);
    }

    // Partial tiles.  Wave v adds, in wave order, block row v / 2,
    // registers 8 (v % 2) .. + 7 of both blocks j (16 values per lane), and
    // stores them.  Each wave writes its partial into its own stages, which
    // no other wave reads and which hold no copy in flight after its last
    // phase (so no barrier is needed before): slot v holds what wave v adds,
    // as groups g = 2 j + h (registers 8 (v % 2) + 4 h .. + 3 of block (v /
    // 2, j)), lane l's four values at word v SLOT + 4 (64 g + l): one 128-bit
    // write or read per group, consecutive lanes on consecutive 16 bytes.
    // Register r of lane (li, lh) is row rho = 8 (r / 4) + 4 lh + r % 4 of
    // its block (tile row 32 i + rho for a k-contiguous A, 2 rho + i for an
    // mn-contiguous one) and column li (32 j + li, or 2 li + j: then the two
    // blocks' values are adjacent columns, one 64-bit store; N is a multiple
    // of 4, so both are in or out).
    constexpr int SLOT = 4 * 4 * 64;
    static_assert(4 * SLOT <= WAVE_WORDS, "slots fit in the wave's stages");
    {
        float* const mine = lds + w * WAVE_WORDS;
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 8 * (v & 1) + 4 * h;
                    const floatx4 x = {acc[v >> 1][j][r], acc[v >> 1][j][r + 1], acc[v >> 1][j][r + 2],
                                       acc[v >> 1][j][r + 3]};
                    *reinterpret_cast<floatx4*>(mine + v * SLOT + 4 * (64 * (2 * j + h) + lane)) = x;
                }
    }
    __syncthreads();
    mark(3);
    const int bi = w >> 1, r0 = 8 * (w & 1);
    floatx4 sum[FN][2];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const floatx4 x =
                    *reinterpret_cast<const floatx4*>(lds + u * WAVE_WORDS + w * SLOT + 4 * (64 * (2 * j + h) + lane));
                if (u == 0) sum[j][h] = x;
                else sum[j][h] += x;
            }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int r = r0 + rr;
        const int rho = 8 * (r >> 2) + 4 * lh + (r & 3);
        const int row = m0 + (KCA ? 32 * bi + rho : FM * rho + bi);
        if (row >= p.M) continue;
        float* crow = p.C + (int64_t)row * p.ldc + n0;
        if constexpr (!KCB) {
            if (n0 + 2 * li < p.N) {
                const floatx2 x = {sum[0][rr >> 2][rr & 3], sum[1][rr >> 2][rr & 3]};
                *reinterpret_cast<floatx2*>(crow + 2 * li) = x;
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                if (n0 + 32 * j + li < p.N) crow[32 * j + li] = sum[j][rr >> 2][rr & 3];
        }
    }
    if constexpr (TL) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        mark(4);
        if (lane == 0 && (int)blockIdx.x < timeline_blocks) {
            uint32_t* o = timeline + 8 * (4 * (int64_t)blockIdx.x + w);
            for (int i = 0; i < 5; ++i) o[i] = tl[i];
            o[5] = tl_cycles;
            o[6] = (uint32_t)P;
            o[7] = blockIdx.x;
        }
    }
}

// 64 x 64 tiles of 2 x 2 waves, each one 32 x 32 block over the whole K,
// from NST (2, 3 or 4) LDS stages of 16 KB in the four-wave schedule's
// layouts.  Phase ph reads stage ph % NST and, after its barrier, copies
// phase ph + NST into that stage.  Several blocks share a CU -- four with
// two stages, three with three (the configuration the tile choice runs),
// two with four -- so one block's start, end and waits overlap the others'
// work, and the copies run NST - 1 phases ahead (a phase is only 16 matrix
// instructions, about 1000 clocks).  The barrier of phase ph comes
// between steps 2 and 3, once every wave's copies of phase ph + 1 have
// landed and its reads of phase ph's fragments have completed; it is the
// bare s_barrier, as a fence would also wait for the copies of later
// phases.  Every phase issues the four copies of phase ph + NST, past the
// end (zeros into a stage nothing reads) when there is no such phase, so the
// wait before the barrier is always for all but the last 4 (NST - 2)
// copies.  The loop is unrolled by the stages (each stage's offset an
// instruction offset); two accumulators take the even and odd instructions
// of a step (none waits for the one before), added at the end; the last
// phase skips its 8-deep steps wholly at k >= K.
template <bool KCA, bool KCB, int NST>
__global__ __launch_bounds__(256)
void gemm_f32_tile64_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    static_assert(NST >= 2 && NST <= 4, "stages");
    constexpr int BM = 64, BN = 64, WM = 32, WN = 32, NMFMA = 4;
    using TA = SchedTileF32<KCA, BM, 1>;
    using TB = SchedTileF32<KCB, BN, 1>;
    constexpr int A_COPIES = TA::COPIES, NCOPY = TA::COPIES + TB::COPIES;
    constexpr int NREAD = TA::READS + TB::READS;          // 2, 5 or 8
    constexpr int RPS = (NREAD + NMFMA - 1) / NMFMA;      // reads after each matrix instruction
    static_assert(NCOPY == NMFMA && NREAD <= RPS * NMFMA && RPS <= 2, "schedule");
    constexpr int A_ST = TA::WORDS, B_ST = TB::WORDS;    // floats per stage
    __shared__ __attribute__((aligned(16))) float lds[NST * (A_ST + B_ST)];   // A's stages, then B's

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave_u / 2, wn = wave_u % 2;
    const int li = lane & 31, lh = lane >> 5;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    // Copies 0, 1 fill A's tile, 2, 3 B's; descriptors and zeros as in
    // gemm_f32_sched_kernel (the last phase's offsets hold the phase, lanes
    // at k >= K point past the end).
    uint32_t doff[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        doff[j] = TA::copy_src(wave_u, j, lane, m0, p.lda);
        doff[A_COPIES + j] = TB::copy_src(wave_u, j, lane, n0, p.ldb);
    }
    constexpr int kRawBufferWord3 = 0x00020000;
    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.A), (short)0, (int)(4 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.B), (short)0, (int)(4 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    const int P = ceil_div(p.K, kSBK);
    constexpr uint32_t kPastEnd = 0x80000000u;
    const int klast = (P - 1) * kSBK;
    uint32_t dlast[NCOPY];
#pragma unroll
    for (int j = 0; j < A_COPIES; ++j) {
        const int ka = klast + TA::copy_k(wave_u, j, lane);
        const int kb = klast + TB::copy_k(wave_u, j, lane);
        dlast[j] = ka >= p.K ? kPastEnd : doff[j] + (uint32_t)TA::phase_bytes(klast, p.lda);
        dlast[A_COPIES + j] = kb >= p.K ? kPastEnd : doff[A_COPIES + j] + (uint32_t)TB::phase_bytes(klast, p.ldb);
    }
    // Per-lane and scalar offsets of the copies of phase ph (any ph >= 0).
    uint32_t cv[NCOPY];
    int cs_a = 0, cs_b = 0;
    auto plan = [&](int ph) __attribute__((always_inline)) {
        const bool normal = ph < P - 1, last = ph == P - 1;
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) cv[j] = normal ? doff[j] : (last ? dlast[j] : kPastEnd);
        cs_a = normal ? TA::phase_bytes(ph * kSBK, p.lda) : 0;
        cs_b = normal ? TB::phase_bytes(ph * kSBK, p.ldb) : 0;
    };
    auto copy = [&](int j, int st) __attribute__((always_inline)) {
        if (j < A_COPIES) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(lds + st * A_ST + TA::copy_dst(wave_u, j)), 16,
                (int)cv[j], cs_a, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b,
                (__attribute__((address_space(3))) void*)(lds + NST * A_ST + st * B_ST +
                                                         TB::copy_dst(wave_u, j - A_COPIES)),
                16, (int)cv[j], cs_b, 0, 0);
        }
    };

    // Read bases (stage 0): KC one per step, MC one in all; the stage and
    // the read are instruction offsets.
    constexpr int SA = KCA ? 4 : 1, SB = KCB ? 4 : 1;
    uint32_t abase[SA], bbase[SB];
    const uint32_t lds0 = lds_addr(lds);
#pragma unroll
    for (int s = 0; s < SA; ++s) abase[s] = lds0 + TA::read_base(wm * WM, s, li, lh);
#pragma unroll
    for (int s = 0; s < SB; ++s) bbase[s] = lds0 + 4u * NST * A_ST + TB::read_base(wn * WN, s, li, lh);

    // A fragment is one floatx4 either way: a k-contiguous one read whole,
    // an mn-contiguous one value i of its four reads (k rows apart), so the
    // reads land where the instructions take them (value e for instruction
    // e) and no register move waits for them.
    floatx4 a[2][1], b[2][1];
    auto read_one = [&](auto tile, floatx4 (&x)[1], uint32_t base, int s, int i, int st) __attribute__((always_inline)) {
        using T = decltype(tile);
        const uint32_t addr = base + T::read_imm(s, i) + 4u * st * T::WORDS;
        if constexpr (T::IS_KC) x[0] = lds_read128(addr);
        else x[0][i] = *(volatile const __attribute__((address_space(3))) float*)(uintptr_t)addr;   // unmerged
    };
    auto read_op = [&](int s, int t, int i, int st) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, a[t], abase[KCA ? s : 0], s, i, st);
        else read_one(TB{}, b[t], bbase[KCB ? s : 0], s, i - TA::READS, st);
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[t][0]), "+v"(b[t][0]) : : "memory");
    };

    floatx16 acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[h][r] = 0.0f;

    using yes = std::true_type;
    using no = std::false_type;
    // One step on set t: instruction e on accumulator e % 2; after it, reads
    // RPS e .. of step rs (stage rst) into set t ^ 1 if R, and copy e into
    // stage cst if C.
    auto step = [&](int t, auto reads, int rs, int rst, auto copies, int cst) __attribute__((always_inline)) {
        constexpr bool R = decltype(reads)::value;
        constexpr bool C = decltype(copies)::value;
        unroll<NMFMA>([&](auto qc) __attribute__((always_inline)) {
            constexpr int e = decltype(qc)::value;
            acc[e & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t][0][e], b[t][0][e], acc[e & 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (R && RPS * e < NREAD) {
                read_op(rs, t ^ 1, RPS * e, rst);
                if constexpr (RPS == 2 && RPS * e + 1 < NREAD) read_op(rs, t ^ 1, RPS * e + 1, rst);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (C) {
                copy(e, cst);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    // The barrier alone: each wave has waited for its own copies, and a
    // fence here would make the compiler wait for every copy in flight.
    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Prologue: phases 0 .. NST - 1 into stages 0 .. NST - 1 (past the end
    // beyond P - 1), then wait for phase 0 (all but the last 4 (NST - 1)
    // copies).
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        plan(st);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) copy(j, st);
    }
    if constexpr (NST == 4) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (NST == 3) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    barrier();
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(0, 0, i, 0);
    __builtin_amdgcn_sched_barrier(0);

    // Phase ph on stage ST.  Steps that run: all but in the last phase,
    // where only those holding some k < K.
    auto phase = [&](auto stc, int ph) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value, NX = (ST + 1) % NST;
        const int steps = ph == P - 1 ? (p.K - klast + 7) / 8 : 4;
        wait_set(0);
        step(0, yes{}, 1, ST, no{}, 0);
        wait_set(1);
        if (steps > 1) {
            step(1, yes{}, 2, ST, no{}, 0);
            wait_set(0);
            if (steps > 2) {
                step(0, yes{}, 3, ST, no{}, 0);
                wait_set(1);
            }
        }
        plan(ph + NST);
        if constexpr (NST == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // this wave's copies of phase ph + 1
        else if constexpr (NST == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
        if (steps > 3) step(1, yes{}, 0, NX, yes{}, ST);    // reads step 0 of phase ph + 1
        else {
#pragma unroll
            for (int j = 0; j < NCOPY; ++j) copy(j, ST);   // the count of copies stays four per phase
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    int ph = 0;
    for (; ph + NST <= P; ph += NST)
        unroll<NST>([&](auto stc) __attribute__((always_inline)) { phase(stc, ph + decltype(stc)::value); });
    unroll<NST - 1>([&](auto stc) __attribute__((always_inline)) {
        if (ph < P) phase(stc, ph++);
    });
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // the dummy copies, before the block ends

#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] += acc[1][r];
    // Guarded store: register r of lane (li, lh) is row 8 (r / 4) + 4 lh + r
    // % 4 and column li of the wave's block.
    const int col = n0 + wn * WN + li;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = acc[0][r];
    }
}

template <bool KCA, bool KCB>
hipError_t launch_ksplit_f32_kernel(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                    unsigned blocks) {
    hipLaunchKernelGGL((gemm_f32_ksplit_kernel<KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m, nullptr, 0);
    return hipGetLastError();
}

template <int F, bool KCA, bool KCB>
hipError_t launch_sched_f32_kernel(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                   unsigned blocks) {
    hipLaunchKernelGGL((gemm_f32_sched_kernel<F, F, KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

template <int F>
hipError_t launch_sched_f32_tile(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m) {
    constexpr int T = 64 * F;
    const int tiles_m = ceil_div(p.M, T), tiles_n = ceil_div(p.N, T);
    const unsigned blocks = (unsigned)((int64_t)tiles_m * tiles_n);
    switch (2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_sched_f32_kernel<F, true, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 1: return launch_sched_f32_kernel<F, true, true>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 2: return launch_sched_f32_kernel<F, false, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        default: return launch_sched_f32_kernel<F, false, true>(p, s, tiles_m, tiles_n, group_m, blocks);
    }
}
}  // namespace

// K, M and N multiples of 4 (edge tiles and a last phase past K run whole,
// see the descriptors above).  Any leading dimension and dword alignment will do:
// gfx9 runs memory in unaligned-access mode, so the 16-byte copies and
// stores need only the 4-byte alignment the entry points check.
bool sched_f32_fits(const GemmArgs& p, int op_a, int op_b) {
    if (p.K % 4 != 0 || p.K <= 0 || p.M % 4 != 0 || p.N % 4 != 0) return false;
    // A stored M x K (op N) or K x M (op T); B stored K x N or N x K.  Byte
    // offsets, edge tiles' overhang included, stay below 2^31.
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const int64_t lim = (int64_t)1 << 31;
    return 4 * (a_rows + 256) * p.lda < lim && 4 * (b_rows + 256) * p.ldb < lim;
}

// K, M and N multiples of 4 (see the descriptors of the kernel), stored
// factors below 2^31 bytes with a tile's overhang.
bool ksplit_f32_fits(const GemmArgs& p, int op_a, int op_b) {
    if (p.K % 4 != 0 || p.K <= 0 || p.M % 4 != 0 || p.N % 4 != 0) return false;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const int64_t lim = (int64_t)1 << 31;
    return 4 * (a_rows + 256) * p.lda < lim && 4 * (b_rows + 256) * p.ldb < lim;
}

// The product's k-split launch (A and B as stored) on its measurement
// instantiation, which also records the timeline described at the kernel.
hipError_t launch_ksplit_f32_timeline(const GemmArgs& p, hipStream_t s, int group_m, uint32_t* timeline,
                                      int timeline_blocks) {
    const int tiles_m = ceil_div(p.M, 64), tiles_n = ceil_div(p.N, 64);
    const unsigned blocks = (unsigned)((int64_t)tiles_m * tiles_n);
    hipLaunchKernelGGL((gemm_f32_ksplit_kernel<true, false, true>), dim3(blocks), dim3(256), 0, s, p, tiles_m,
                       tiles_n, group_m, timeline, timeline_blocks);
    return hipGetLastError();
}

hipError_t launch_ksplit_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m) {
    const int tiles_m = ceil_div(p.M, 64), tiles_n = ceil_div(p.N, 64);
    const unsigned blocks = (unsigned)((int64_t)tiles_m * tiles_n);
    switch (2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_ksplit_f32_kernel<true, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 1: return launch_ksplit_f32_kernel<true, true>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 2: return launch_ksplit_f32_kernel<false, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        default: return launch_ksplit_f32_kernel<false, true>(p, s, tiles_m, tiles_n, group_m, blocks);
    }
}

template <int NST>
hipError_t launch_tile64_stages(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m) {
    const int tiles_m = ceil_div(p.M, 64), tiles_n = ceil_div(p.N, 64);
    const dim3 grid((unsigned)((int64_t)tiles_m * tiles_n)), block(256);
    switch (2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: hipLaunchKernelGGL((gemm_f32_tile64_kernel<true, false, NST>), grid, block, 0, s, p, tiles_m, tiles_n, group_m); break;
        case 1: hipLaunchKernelGGL((gemm_f32_tile64_kernel<true, true, NST>), grid, block, 0, s, p, tiles_m, tiles_n, group_m); break;
        case 2: hipLaunchKernelGGL((gemm_f32_tile64_kernel<false, false, NST>), grid, block, 0, s, p, tiles_m, tiles_n, group_m); break;
        default: hipLaunchKernelGGL((gemm_f32_tile64_kernel<false, true, NST>), grid, block, 0, s, p, tiles_m, tiles_n, group_m); break;
    }
    return hipGetLastError();
}

hipError_t launch_tile64_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m, int stages) {
    if (stages == 4) return launch_tile64_stages<4>(p, s, op_a, op_b, group_m);
    if (stages == 3) return launch_tile64_stages<3>(p, s, op_a, op_b, group_m);
    return launch_tile64_stages<2>(p, s, op_a, op_b, group_m);
}

hipError_t launch_sched_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m, int tile) {
    return tile == 128 ? launch_sched_f32_tile<2>(p, s, op_a, op_b, group_m)
                       : launch_sched_f32_tile<4>(p, s, op_a, op_b, group_m);
}

}  // namespace gemmf32
