// mfma_ksplit96.hip -- rung 3 on 96 x 96 output tiles whose four waves
// split the tile's phases.
//
// The tiled product of the pages' shared-memory chapter (PMPP chapter 5
// notes, sections 5.4-5.5: per phase the tiles of A and B are staged in
// shared memory, the multiply-adds run from them, ghost elements past the
// matrix edges are zeros, and the store is guarded), for the shapes whose
// 64 x 64, 128 x 128 and 256 x 256 tiles fill the 256 CUs badly: 1536^3 has
// 576 tiles of 64 x 64 (2.25 rounds) but 256 of 96 x 96 (one), 7168^3 5625
// of 96 x 96 (22 rounds, the last one nearly full).
//
// One tile per block.  Each of the four waves (one per SIMD) computes the
// whole tile -- 3 x 3 blocks of 32 x 32 on v_mfma_f32_32x32x2_f32, 144
// accumulator registers -- over every fourth 16-deep phase (wave w: phases
// w, w + 4, ...), from two LDS stages of its own (14 KB each) that only it
// copies into (direct global -> LDS copies) and reads, so no wave waits for
// another before the end, where the four partial tiles are added in wave
// order through LDS (deterministic; the same bits for every op pair).  A
// phase is two steps of 36 instructions (8 k each, 4 instructions of 2 k for
// each of the 9 blocks), 4608 matrix-core clocks; a step's instructions are
// followed by the reads of the next step's fragments (one after each of the
// first), and the second step's, after its reads, by the 14 copies of the
// phase two ahead into the stage the phase came from (whose reads are all
// done by then).
//
// Tiles (per stage, 96 mn x 16 k):
//   KC (k-contiguous factor: A as stored, B stored transposed): 96 rows of
//      16 k (64 bytes), the 16-byte chunk c (4 k) of row r at
//      c ^ ((r / 4) mod 4); a 1 KB copy fills 16 rows (6 copies).  Lane l
//      reads, for block f and step s, the 128 bits of row 32 f + l % 32,
//      k = 8 s + 4 (l / 32) .. + 3: value e is its operand of the step's
//      instruction e.  The 16 lanes of one 128-bit read cycle (4-lane quads
//      of one half-wave by index parity) reach 16 different 4-bank groups.
//   MC (mn-contiguous factor: B as stored, A stored transposed): 16 k rows
//      of 96 values at a 512-byte stride; a 1 KB copy fills 2 rows (8
//      copies; the lanes of the 128 pad bytes copy nothing).  Lane l reads,
//      for block f, step s and instruction e, the 32 bits of k row
//      8 s + 4 (l / 32) + e, column 32 f + l % 32: 32 consecutive words.
// Block f holds rows (or columns) 32 f .. 32 f + 31 of the tile either way.
//
// Edges and K as in the 64 x 64 k-split kernel (mfma_sched.hip): K, M and
// N multiples of 4; phases aligned to the end of K, so only phase 0 reaches
// below k = 0; every copy that must bring zeros is past its descriptor's
// end by its per-lane offset alone (rows of a KC factor past the tile's
// edge, chunks of an MC factor past its last column, lanes of phase 0 below
// k = 0, positions holding no phase).  Each wave takes its phases in the
// order P - 1, (a position copying zeros if P is odd,) 0, 1, .., P - 2: the
// two phases that need per-lane offsets -- the last (an MC factor's last
// row, across its last column, must meet the descriptor's end by its own
// offset) and the first -- are copied in the prologue and by the first two
// phases, so the phase loop has one body with one kind of copy (a branch
// between phases would keep an unread register set live across it).
#include "launch.h"

#include <type_traits>
#include <utility>

namespace gemmf32 {

namespace {

template <typename F, int... Q>
__device__ __forceinline__ void unroll96(F&& f, std::integer_sequence<int, Q...>) {
    (f(std::integral_constant<int, Q>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll_n(F&& f) {
    unroll96(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ floatx4 lds_load128(uint32_t lds_byte_addr) {
    typedef const __attribute__((address_space(3))) floatx4 lds_floatx4;
    return *(lds_floatx4*)(uintptr_t)lds_byte_addr;
}
__device__ __forceinline__ float lds_load32(uint32_t lds_byte_addr) {
    typedef const __attribute__((address_space(3))) float lds_float;
    return *(lds_float*)(uintptr_t)lds_byte_addr;
}
__device__ __forceinline__ uint32_t lds_byte(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Waits for all outstanding LDS reads; the fragments pass through the wait
// as operands, so no use of them is scheduled before it.
__device__ __forceinline__ void wait_frags(floatx4 (&x)[3]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]) : : "memory");
}

template <bool KC>
struct Ksplit96Tile {
    static constexpr int BYTES = KC ? 6144 : 8192;       // per stage
    static constexpr int COPIES = KC ? 6 : 8;            // 1 KB copies per phase
    static constexpr int READS = KC ? 3 : 12;            // LDS reads per step
    static constexpr bool IS_KC = KC;
    // Copy j, lane l: the stored row (KC: mn; MC: k) and its first float
    // (KC: k; MC: mn) relative to the tile and phase; LDS byte 1024 j + 16 l.
    __host__ __device__ static int copy_row(int j, int lane) { return KC ? 16 * j + lane / 4 : 2 * j + lane / 32; }
    __host__ __device__ static int copy_col(int j, int lane) {
        return KC ? 4 * ((lane % 4) ^ ((copy_row(j, lane) >> 2) & 3)) : 4 * (lane % 32);
    }
    __host__ __device__ static int copy_k(int j, int lane) { return KC ? copy_col(j, lane) : copy_row(j, lane); }
    __host__ __device__ static int copy_mn(int j, int lane) { return KC ? copy_row(j, lane) : copy_col(j, lane); }
    // Byte offset of those 4 values from the stored matrix's base at k = 0.
    __host__ __device__ static int64_t copy_src(int j, int lane, int mn0, int64_t ld) {
        return KC ? 4 * ((int64_t)(mn0 + copy_row(j, lane)) * ld + copy_k(j, lane))
                  : 4 * ((int64_t)copy_row(j, lane) * ld + mn0 + copy_mn(j, lane));
    }
    __host__ __device__ static int64_t phase_bytes(int k0, int64_t ld) { return KC ? 4 * (int64_t)k0 : 4 * (int64_t)k0 * ld; }
    // Read base of lane l (bytes from the stage) and the instruction offset
    // of its read for block f, step s and (MC) instruction e:
    //   KC: row 32 f + l % 32, chunk 2 s + l / 32 (the swizzle depends on l % 32)
    //   MC: k row 8 s + 4 (l / 32) + e, column 32 f + l % 32
    __host__ __device__ static uint32_t read_base(int lane) {
        const int li = lane & 31, lh = lane >> 5;
        return KC ? (uint32_t)(64 * li) : (uint32_t)(2048 * lh + 4 * li);
    }
    __host__ __device__ static uint32_t read_chunk(int s, int lane) {   // KC only: per step
        const int li = lane & 31, lh = lane >> 5;
        return (uint32_t)(16 * ((2 * s + lh) ^ ((li >> 2) & 3)));
    }
    __host__ __device__ static constexpr uint32_t read_imm(int f, int s, int e) {
        return KC ? 2048u * f : 4096u * s + 512u * e + 128u * f;
    }
};

template <bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm_f32_ksplit96_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
    using TA = Ksplit96Tile<KCA>;
    using TB = Ksplit96Tile<KCB>;
    constexpr int BK = 16;                               // k per phase
    constexpr int STAGE = TA::BYTES + TB::BYTES;         // bytes per stage
    constexpr int REGION = 36864;                        // per wave: two stages, then its partial tile
    static_assert(2 * STAGE <= REGION, "stages fit in the wave's region");
    constexpr int NA = TA::COPIES, NC = TA::COPIES + TB::COPIES;   // copies per phase
    constexpr int NREAD = TA::READS + TB::READS;         // 6 .. 24 per step
    constexpr int CFIRST = 36 - NC;                      // copies after instructions CFIRST .. 35
    static_assert(NREAD <= 36 && CFIRST >= 0, "schedule");
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * REGION];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * 96;
    const int n0 = (in_g / gm) * 96;

    // This wave's phases: local phase lp is phase 4 lp + w, at k0 = kof(lp).
    // Positions 0 .. P2 - 1 hold phase P - 1, then (with P odd) none, then
    // phases 0, 1, .., P - 2; at least two positions.
    const int nph = (p.K + BK - 1) / BK;
    const int kbase = p.K - BK * nph;                    // -12 .. 0, a multiple of 4
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
        const_cast<float*>(p.A), (short)0, (int)(4 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.B), (short)0, (int)(4 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    // Copies 0 .. NA - 1 fill A's tile, the rest B's.  Chunks of an MC factor
    // in the pad or past its last column point past the end in every phase.
    uint32_t doff[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const bool is_a = j < NA;
        const int jj = is_a ? j : j - NA;
        if (is_a) {
            doff[j] = (uint32_t)TA::copy_src(jj, lane, m0, p.lda);
            if (!KCA && (TA::copy_mn(jj, lane) >= 96 || m0 + TA::copy_mn(jj, lane) >= a_cols)) doff[j] = kPastEnd;
        } else {
            doff[j] = (uint32_t)TB::copy_src(jj, lane, n0, p.ldb);
            if (!KCB && (TB::copy_mn(jj, lane) >= 96 || n0 + TB::copy_mn(jj, lane) >= b_cols)) doff[j] = kPastEnd;
        }
    }
    unsigned char* const wl = lds + w * REGION;
    auto copy_at = [&](int j, uint32_t voff, int soff, int stage) __attribute__((always_inline)) {
        if (j < NA) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + 1024 * j), 16, (int)voff, soff,
                0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + TA::BYTES + 1024 * (j - NA)),
                16, (int)voff, soff, 0, 0);
        }
    };
    // Copy j of the phase at position s >= 4 (phase s - 1 - odd, in 2 ..
    // P - 2: the phase in the scalar offset) into `stage`; positions from
    // P2 on copy into stages nothing reads afterwards.
    auto copy = [&](int j, int s, int stage) __attribute__((always_inline)) {
        const int k0 = kof(s - 1 - odd);
        copy_at(j, doff[j], (int)(j < NA ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb)), stage);
    };
    // Copy j of the phase at position s with the phase in each lane's offset
    // (scalar offset 0): lanes below k = 0 or at k >= K, chunks past an MC
    // factor's edge, and positions holding no phase point past the end.
    auto copy_folded = [&](int j, int s, int stage) __attribute__((always_inline)) {
        const int lp = phase_at(s);
        const int k0 = kof(lp);
        const int kl = j < NA ? TA::copy_k(j, lane) : TB::copy_k(j - NA, lane);
        const int64_t pb = j < NA ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb);
        const bool inside = lp >= 0 && lp < P && k0 + kl >= 0 && k0 + kl < p.K && doff[j] != kPastEnd;
        copy_at(j, inside ? (uint32_t)((int64_t)doff[j] + pb) : kPastEnd, 0, stage);
    };

    // Read bases (bytes, stage 0): KC one per step, MC one; the block, step,
    // instruction and stage are instruction offsets.
    const uint32_t wl0 = lds_byte(wl);
    uint32_t abase[2], bbase[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        abase[s] = wl0 + TA::read_base(lane) + (KCA ? TA::read_chunk(s, lane) : 0u);
        bbase[s] = wl0 + (uint32_t)TA::BYTES + TB::read_base(lane) + (KCB ? TB::read_chunk(s, lane) : 0u);
    }

    // Fragments, two sets (one per step): block f's four operands of the
    // step's instructions e = 0..3.
    floatx4 a[2][3], b[2][3];
    // Read i of step s of the phase in stage STG into set t: A's reads first
    // (KC: block i; MC: block i / 4, instruction i % 4), then B's.
    auto read_op = [&](auto stg, int s, int t, int i) __attribute__((always_inline)) {
        constexpr uint32_t SOFF = (uint32_t)STAGE * decltype(stg)::value;
        if (i < TA::READS) {
            if constexpr (KCA) a[t][i] = lds_load128(abase[s] + SOFF + TA::read_imm(i, s, 0));
            else a[t][i / 4][i % 4] = lds_load32(abase[0] + SOFF + TA::read_imm(i / 4, s, i % 4));
        } else {
            const int r = i - TA::READS;
            if constexpr (KCB) b[t][r] = lds_load128(bbase[s] + SOFF + TB::read_imm(r, s, 0));
            else b[t][r / 4][r % 4] = lds_load32(bbase[0] + SOFF + TB::read_imm(r / 4, s, r % 4));
        }
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        wait_frags(a[t]);
        wait_frags(b[t]);
    };

    floatx16 acc[3][3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One step on set t: instruction q = 9 e + 3 i + j is block (i, j)'s
    // instruction e; after instruction q < NREAD, read q of (next) into set
    // t ^ 1 (RS: its step, STG: its stage); after instruction q >= CFIRST, if
    // C, copy q - CFIRST of position cs into stage cstage (FOLDED: per-lane
    // offsets).
    auto step = [&](int t, auto stg, int rs, auto cc, auto foldc, int cs, int cstage) __attribute__((always_inline)) {
        constexpr bool C = decltype(cc)::value;
        unroll_n<36>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            constexpr int e = q / 9, i = (q / 3) % 3, j = q % 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t][i][e], b[t][j][e], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (q < NREAD) {
                read_op(stg, rs, t ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (C && q >= CFIRST) {
                if constexpr (decltype(foldc)::value) copy_folded(q - CFIRST, cs, cstage);
                else copy(q - CFIRST, cs, cstage);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    using yes = std::true_type;
    using no = std::false_type;
    // The phase at position s in stage U = s % 2: step 0 (set 0; reads step 1
    // from stage U into set 1), then, once the copies of position s + 1 have
    // landed (nothing else in flight), step 1 (set 1; reads step 0 of
    // position s + 1 from stage U ^ 1 into set 0, then copies position s + 2
    // into stage U, whose reads are done).
    auto phase = [&](auto uc, int s, auto foldc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        using CUR = std::integral_constant<int, U>;
        using NXT = std::integral_constant<int, U ^ 1>;
        wait_set(0);
        step(0, CUR{}, 1, no{}, no{}, 0, 0);
        wait_set(1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        step(1, NXT{}, 0, yes{}, foldc, s + 2, U);
    };
    using s0 = std::integral_constant<int, 0>;
    using s1 = std::integral_constant<int, 1>;

#pragma unroll
    for (int j = 0; j < NC; ++j) copy_folded(j, 0, 0);
#pragma unroll
    for (int j = 0; j < NC; ++j) copy_folded(j, 1, 1);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NC) : "memory");           // position 0 has landed
#pragma unroll
    for (int i = 0; i < NREAD; ++i) read_op(s0{}, 0, 0, i);
    __builtin_amdgcn_sched_barrier(0);
    phase(s0{}, 0, yes{});
    __builtin_amdgcn_sched_barrier(0);
    phase(s1{}, 1, yes{});
    __builtin_amdgcn_sched_barrier(0);
    for (int pos = 2; pos < P2; pos += 2) {
        phase(s0{}, pos, no{});
        __builtin_amdgcn_sched_barrier(0);
        phase(s1{}, pos + 1, no{});
        __builtin_amdgcn_sched_barrier(0);
    }
    // the reads of a position past the last, and the copies aimed past it,
    // complete before the region is reused
    wait_set(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Partial tiles.  Register r of block (i, j) is x = 16 (3 i + j) + r;
    // lane l's values x = 4 h .. 4 h + 3 go to byte 1024 h + 16 l of the
    // wave's own region (its stages, done with).  After the barrier wave v
    // adds, in wave order, x = 36 v .. 36 v + 35 of the four partials and
    // stores them: register r of block (i, j) of lane (li, lh) is row
    // 32 i + 8 (r / 4) + 4 lh + r % 4, column 32 j + li of the tile.
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const floatx4 v = {acc[i][j][4 * h], acc[i][j][4 * h + 1], acc[i][j][4 * h + 2], acc[i][j][4 * h + 3]};
                *reinterpret_cast<floatx4*>(wl + 1024 * (4 * (3 * i + j) + h) + 16 * lane) = v;
            }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int hh = 0; hh < 9; ++hh) {
        const int h = 9 * w + hh;                        // group of four registers
        floatx4 sum = *reinterpret_cast<const floatx4*>(lds + 1024 * h + 16 * lane);
#pragma unroll
        for (int u = 1; u < 4; ++u) sum += *reinterpret_cast<const floatx4*>(lds + u * REGION + 1024 * h + 16 * lane);
        const int blk = h >> 2, i = blk / 3, j = blk % 3, r0 = 4 * (h & 3);
        const int col = n0 + 32 * j + li;
        if (col >= p.N) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = r0 + t;
            const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (row < p.M) p.C[(int64_t)row * p.ldc + col] = sum[t];
        }
    }
}

template <bool KCA, bool KCB>
hipError_t launch_ksplit96_kernel(const GemmArgs& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                  unsigned blocks) {
    hipLaunchKernelGGL((gemm_f32_ksplit96_kernel<KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

}  // namespace

// K, M and N multiples of 4, stored factors below 2^31 bytes with a tile's
// overhang.
bool ksplit96_f32_fits(const GemmArgs& p, int op_a, int op_b) {
    if (p.K % 4 != 0 || p.K <= 0 || p.M % 4 != 0 || p.N % 4 != 0) return false;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const int64_t lim = (int64_t)1 << 31;
    return 4 * (a_rows + 128) * p.lda < lim && 4 * (b_rows + 128) * p.ldb < lim;
}

hipError_t launch_ksplit96_f32(const GemmArgs& p, hipStream_t s, int op_a, int op_b, int group_m) {
    const int tiles_m = (p.M + 95) / 96, tiles_n = (p.N + 95) / 96;
    const unsigned blocks = (unsigned)((int64_t)tiles_m * tiles_n);
    switch (2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_ksplit96_kernel<true, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 1: return launch_ksplit96_kernel<true, true>(p, s, tiles_m, tiles_n, group_m, blocks);
        case 2: return launch_ksplit96_kernel<false, false>(p, s, tiles_m, tiles_n, group_m, blocks);
        default: return launch_ksplit96_kernel<false, true>(p, s, tiles_m, tiles_n, group_m, blocks);
    }
}

}  // namespace gemmf32
