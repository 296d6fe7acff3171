// mfma16_ksplit.hip -- the mixed-precision product (bfloat16 or binary16
// factors, binary32 accumulation) for few output tiles and long K.
//
// The one-volume PMPP notes run the fully connected layer as a matrix
// product on matrix units fed FP16 or BF16 and accumulating in FP32
// (deep-learning chapter, "FC Layer = GEMM", "Mixed Precision"); this is
// that product with the tiled structure of the pages' shared-memory chapter
// (tiles staged in LDS, ghost zeros past the matrix edges, a guarded store),
// for the shapes whose large tiles would leave most compute units idle.
//
// Built with the matrix instructions' vector-register form
// (-mllvm -amdgpu-mfma-vgpr-form=true, see build.py): with the accumulators
// in AGPRs the register allocator copied every accumulator before each
// matrix instruction of this kernel.
#include "mfma16_common.h"

namespace gemmf32 {

namespace {

// Few output tiles, long K: 64 x 64 tiles, one per block, whose four waves
// each compute the whole tile over every fourth 32-deep phase (wave w:
// phases w, w + 4, ...) from LDS stages of their own, which only that wave
// copies into and reads; the four partial tiles meet in LDS at the end and
// are added in wave order (deterministic; the same bits for every op pair).
// A 1024 x 1024 x 4096 product has 16 tiles of 256 x 256 for 256 CUs; here
// it has 256 blocks.
//
// Matrix instruction v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies
// A[l % 16][8 (l / 16) .. + 7] and B[8 (l / 16) .. + 7][l % 16]; accumulator
// register r holds D[4 (l / 16) + r][l % 16].  A wave's 64 x 64 tile is 4 x 4
// blocks of 16 x 16; a 32-deep phase is one step of 16 instructions, about
// 256 clocks of the matrix core, so each wave keeps four stages (8 KB each,
// 128 KB per block) and copies a phase three phases ahead of its use.  The
// phase loop is unrolled by the four stages, so every stage offset is an
// instruction offset: besides the matrix instructions the loop holds only
// the fragment reads and the copies (buffer loads into LDS whose phase is in
// the scalar offset).
//
// Tiles (per stage):
//   KC (k-contiguous factor: A as stored, B stored transposed): 64 rows of
//      32 k (64 bytes), the 16-byte chunk c (8 k) of row r at
//      c ^ (2 ((r / 8) mod 2)); a 1 KB copy fills 16 rows; a fragment is one
//      128-bit read of row 16 f + l % 16, chunk l / 16.  A 128-bit read
//      serves, per half-wave, the 4-lane quads of even index parity in one
//      cycle (lanes 0-3, 12-15, 20-23, 24-27) and the others in the next
//      (measured on MI355X); those 16 lanes hit 16 different 4-bank groups.
//   MC (mn-contiguous factor: B as stored, A stored transposed): 32 k rows
//      of 64 values (128 bytes), chunk c of row r at
//      c ^ (2 ((r / 2) mod 2) + 4 ((r / 8) mod 2)); a copy fills 8 rows; a
//      fragment is two ds_read_b64_tr_b16 reads (k 0..3 and 4..7 of the lane
//      group's eight), the 32 lanes of one read cycle over 8 rows and 16
//      different 4-bank groups.
//
// Phases are aligned to the end of K (K a multiple of 8), phase g covering
// k = K - 32 (P - g) .. + 31: only phase 0 can reach below k = 0, and its
// lanes there are pointed past the end of their buffer descriptor (zeros).
// Every copy that must bring zeros has a per-lane offset past the
// descriptor's end by itself (the scalar offset, which holds the phase,
// never decides it): rows of a KC factor past the tile's edge, and the
// 16-byte chunks of an MC factor wholly past its last column (in every
// phase).  A chunk of an MC factor across its last column reads the next
// row (only C entries outside the matrix use it), or, in the factor's last
// row -- in the last phase, whose per-lane offsets hold the phase (dlast) --
// its dwords up to the descriptor's end and zeros past it (the range check
// is per dword; the width is even, so no dword straddles the end).
template <bool KC>
struct KsplitTile16 {
    static constexpr int ELEMS = 64 * 32;               // per stage
    static constexpr int CPR = KC ? 4 : 8;               // 16-byte chunks per stored row
    static constexpr int RPC = 64 / CPR;                 // stored rows per 1 KB copy
    static constexpr int ROW = KC ? 32 : 64;             // elements per stored row
    static constexpr int READS = KC ? 4 : 8;             // LDS reads per step (4 fragments)
    static constexpr bool IS_KC = KC;
    __host__ __device__ static constexpr int swz(int r) {
        return KC ? (((r >> 3) & 1) << 1) : ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
    }
    // Copy j (0..3) fills stored rows RPC j .. RPC j + RPC - 1; lane l fills
    // physical chunk l % CPR of row RPC j + l / CPR, so it brings the logical
    // chunk (l % CPR) ^ swz(row).
    __host__ __device__ static int copy_row(int j, int lane) { return RPC * j + lane / CPR; }
    __host__ __device__ static int copy_chunk(int j, int lane) { return (lane % CPR) ^ swz(copy_row(j, lane)); }
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
    // Read base of lane l (bytes from stage 0 of this tile) for block f, and
    // the instruction offset of its read i (KC: i = 0; MC: i = 0, 1).
    //   KC: row 16 f + l % 16, chunk l / 16: 64 (l % 16) + 16 ((l / 16) ^ swz(l % 16)) + 1024 f
    //   MC: rows 8 (l / 16) + 4 i + (l % 16) / 4, values 16 f + 4 (l % 4) .. + 3
    __host__ __device__ static uint32_t read_base(int f, int lane) {
        const int j = lane & 15, g = lane >> 4;
        if constexpr (KC) {
            return (uint32_t)(64 * j + 16 * (g ^ swz(j)));
        } else {
            const int q = j >> 2, jj = j & 3;
            const int r0 = 8 * g + q;
            return (uint32_t)(128 * r0 + 16 * ((2 * f + (jj >> 1)) ^ swz(r0)) + 8 * (jj & 1));
        }
    }
    __host__ __device__ static constexpr uint32_t read_imm(int f, int i) { return KC ? 1024u * f : 512u * i; }
};

template <int FMT, bool KCA, bool KCB>
__global__ __launch_bounds__(256)
void gemm16_ksplit_kernel(Gemm16Args p, int tiles_m, int tiles_n, int group_m) {
    using TA = KsplitTile16<KCA>;
    using TB = KsplitTile16<KCB>;
    constexpr int NS = 4, BK = 32;                       // stages per wave, k per phase
    constexpr int STAGE = TA::ELEMS + TB::ELEMS;         // elements per stage (8 KB)
    constexpr int WAVE_ELEMS = NS * STAGE;               // 32 KB per wave
    constexpr int NREAD = TA::READS + TB::READS;
    static_assert(NREAD <= 16, "one read per matrix instruction at most");
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * WAVE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int logical = xcd_contiguous((int)blockIdx.x, tiles_m * tiles_n);
    const int group_size = group_m * tiles_n;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * group_size;
    const int m0 = (first_m + in_g % gm) * 64;
    const int n0 = (in_g / gm) * 64;

    // This wave's phases: local phase lp is phase 4 lp + w, at k0 = kof(lp).
    const int nph = ceil_div(p.K, BK);
    const int kbase = p.K - BK * nph;                    // -24 .. 0, a multiple of 8
    const int P = nph > w ? (nph - 1 - w) / 4 + 1 : 0;
    auto kof = [&](int lp) __attribute__((always_inline)) { return kbase + BK * (4 * lp + w); };

    const int64_t a_rows = KCA ? p.M : p.K, a_cols = KCA ? p.K : p.M;
    const int64_t b_rows = KCB ? p.N : p.K, b_cols = KCB ? p.K : p.N;
    constexpr int kRawBufferWord3 = 0x00020000;
    constexpr uint32_t kPastEnd = 0x80000000u;           // beyond any descriptor here
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.A), (short)0, (int)(2 * ((a_rows - 1) * p.lda + a_cols)), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.B), (short)0, (int)(2 * ((b_rows - 1) * p.ldb + b_cols)), kRawBufferWord3);
    // Copies 0..3 fill A's tile, 4..7 B's (byte offsets below 2^31: the
    // launcher checks the operands' extents).
    uint32_t doff[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        doff[j] = (uint32_t)TA::copy_src(j, lane, m0, p.lda);
        doff[4 + j] = (uint32_t)TB::copy_src(j, lane, n0, p.ldb);
        if (!KCA && m0 + TA::copy_mn(j, lane) >= a_cols) doff[j] = kPastEnd;
        if (!KCB && n0 + TB::copy_mn(j, lane) >= b_cols) doff[4 + j] = kPastEnd;
    }
    uint16_t* const wl = lds + w * WAVE_ELEMS;
    auto copy_at = [&](int j, uint32_t voff, int soff, int stage) __attribute__((always_inline)) {
        if (j < 4) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + 512 * j), 16, (int)voff, soff,
                0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (__attribute__((address_space(3))) void*)(wl + stage * STAGE + TA::ELEMS + 512 * (j - 4)), 16,
                (int)voff, soff, 0, 0);
        }
    };
    // The wave's last phase (when it is not also its first) takes offsets of
    // its own with the phase folded in and a scalar offset of 0, so that the
    // chunk of an MC factor's last row across its last column meets the
    // descriptor's end by its per-lane offset.
    uint32_t dlast[8];
    {
        const int kl = kof(P > 0 ? P - 1 : 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t pb = j < 4 ? TA::phase_bytes(kl, p.lda) : TB::phase_bytes(kl, p.ldb);
            dlast[j] = doff[j] == kPastEnd ? kPastEnd : (uint32_t)((int64_t)doff[j] + pb);
        }
    }
    // Copy j of local phase lp (k0 >= 0) into its stage; LAST: lp is the
    // wave's last phase.
    auto copy = [&](int j, int lp, int stage, auto lastc) __attribute__((always_inline)) {
        if constexpr (decltype(lastc)::value) {
            copy_at(j, dlast[j], 0, stage);
        } else {
            const int k0 = kof(lp);
            copy_at(j, doff[j], (int)(j < 4 ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb)), stage);
        }
    };
    // The wave's first phase (k0 <= 0 only for phase 0), into stage 0: the
    // phase goes into each lane's offset, lanes below k = 0 point past the end.
    auto copy_first = [&]() __attribute__((always_inline)) {
        const int k0 = kof(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kl = j < 4 ? TA::copy_k(j, lane) : TB::copy_k(j - 4, lane);
            const int64_t pb = j < 4 ? TA::phase_bytes(k0, p.lda) : TB::phase_bytes(k0, p.ldb);
            copy_at(j, k0 + kl >= 0 && doff[j] != kPastEnd ? (uint32_t)((int64_t)doff[j] + pb) : kPastEnd, 0, 0);
        }
    };

    // Read bases (bytes, stage 0); the block and the stage are instruction offsets.
    const uint32_t wl0 = lds_addr(wl);
    uint32_t abase[KCA ? 1 : 4], bbase[KCB ? 1 : 4];
#pragma unroll
    for (int f = 0; f < (KCA ? 1 : 4); ++f) abase[f] = wl0 + TA::read_base(f, lane);
#pragma unroll
    for (int f = 0; f < (KCB ? 1 : 4); ++f) bbase[f] = wl0 + 2u * TA::ELEMS + TB::read_base(f, lane);

    u32x4 a[2][4], b[2][4];
    // Read i (0 .. NREAD - 1) of the phase in stage STG into set x: A's
    // fragments first (KC: read f = fragment f; MC: half i % 2 of fragment
    // i / 2), then B's.
    auto read_one = [&](auto tile, u32x4 (&x)[4], const uint32_t* base, auto stg, int i) __attribute__((always_inline)) {
        using T = decltype(tile);
        constexpr uint32_t SOFF = 2u * STAGE * decltype(stg)::value;
        if constexpr (T::IS_KC) {
            x[i] = lds_read128(base[0] + SOFF + T::read_imm(i, 0));
        } else {
            const int f = i / 2, r = i % 2;
            const u32x2 v = read_tr16_off(base[f], (int)(SOFF + T::read_imm(f, r)));
            x[f][2 * r] = v[0];
            x[f][2 * r + 1] = v[1];
        }
    };
    auto read_op = [&](auto stg, int t, int i) __attribute__((always_inline)) {
        if (i < TA::READS) read_one(TA{}, a[t], abase, stg, i);
        else read_one(TB{}, b[t], bbase, stg, i - TA::READS);
    };
    auto wait_set = [&](int t) __attribute__((always_inline)) {
        wait_tied(a[t]);
        wait_tied(b[t]);
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One phase in stage U % NS, fragments in set U % 2 (U: the phase's
    // position in the unrolled group of NS): its 16 matrix instructions;
    // after instruction q (q < NREAD) read q of the next phase (from stage
    // (U + 1) % NS into the other set) if R, and after every odd one copy
    // q / 2 of local phase lp + 3 into stage (U + 3) % NS if C.
    auto phase = [&](auto uc, int lp, auto rc, auto cc, auto lastc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        constexpr bool R = decltype(rc)::value, C = decltype(cc)::value;
        constexpr int T = U & 1;
        using NEXT = std::integral_constant<int, (U + 1) % NS>;
        unroll<16>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            acc[q / 4][q % 4] = mfma16x16<FMT>(a[T][q / 4], b[T][q % 4], acc[q / 4][q % 4]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (R && q < NREAD) {
                read_op(NEXT{}, T ^ 1, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (C && q % 2 == 1) {
                copy(q / 2, lp + 3, (U + 3) % NS, lastc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (R) wait_set(T ^ 1);
    };
    using yes = std::true_type;
    using no = std::false_type;

    if (P > 0) {
        copy_first();
#pragma unroll
        for (int lp = 1; lp < NS - 1; ++lp) {
            if (lp < P - 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j) copy(j, lp, lp, no{});
            } else if (lp == P - 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j) copy(j, lp, lp, yes{});
            }
        }
        // phase 0 has landed when at most the copies of phases 1 .. min(2, P - 1) are outstanding
        if (P >= 3) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (P == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < NREAD; ++i) read_op(std::integral_constant<int, 0>{}, 0, i);
        wait_set(0);
        __builtin_amdgcn_sched_barrier(0);
        // Full phases in groups of NS (each copies the phase three ahead --
        // never the wave's last one -- and reads the next; the next phase's
        // copies have landed before its reads when at most those of phase
        // lp + 2 are outstanding), then the last ones.
        int lp0 = 0;
        for (; lp0 + NS + 3 < P; lp0 += NS) {
            unroll<NS>([&](auto uc) __attribute__((always_inline)) {
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                phase(uc, lp0 + decltype(uc)::value, yes{}, yes{}, no{});
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        for (; lp0 < P; lp0 += NS) {
            unroll<NS>([&](auto uc) __attribute__((always_inline)) {
                const int lp = lp0 + decltype(uc)::value;
                if (lp < P) {
                    if (lp + 2 < P) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                    if (lp + 3 < P - 1) phase(uc, lp, yes{}, yes{}, no{});
                    else if (lp + 3 == P - 1) phase(uc, lp, yes{}, yes{}, yes{});
                    else if (lp + 1 < P) phase(uc, lp, yes{}, no{}, no{});
                    else phase(uc, lp, no{}, no{}, no{});
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        }
    }

    // Partial tiles: register r of block (i, j) of lane l of wave v at float
    // v 4096 + ((4 i + j) 4 + r) 64 + l.  Wave v then adds, in wave order,
    // block row v: register r of block (v, j) of lane l is row 16 v + 4 (l /
    // 16) + r, column 16 j + l % 16 of the tile.
    __syncthreads();
    float* const part = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[w * 4096 + ((4 * i + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    __syncthreads();
    const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 16 * j + col_l;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float* q = part + ((4 * w + j) * 4 + r) * 64 + lane;
            const float v = ((q[0] + q[4096]) + q[2 * 4096]) + q[3 * 4096];
            const int row = m0 + 16 * w + row_l + r;
            if (row < p.M && col < p.N) p.C[(int64_t)row * p.ldc + col] = v;
        }
    }
}

}  // namespace

// The k-split kernel takes K a multiple of 8, an mn-contiguous factor's
// width even, vector-aligned operands (4-byte aligned bases, even leading
// dimensions) and operands below 2^31 bytes with a tile's overhang (32-bit
// offsets).
bool ksplit16_fits(const Gemm16Args& p, int op_a, int op_b) {
    const bool vec = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 3) == 0 &&
                     (p.lda % 2) == 0 && (p.ldb % 2) == 0;
    const int64_t a_rows = op_a ? p.K : p.M, b_rows = op_b ? p.N : p.K;
    const bool widths = (op_a == 0 || p.M % 2 == 0) && (op_b != 0 || p.N % 2 == 0);
    return vec && widths && p.K % 8 == 0 && p.K > 0 && p.M > 0 && p.N > 0 &&
           2 * (a_rows + 64) * p.lda < (1ll << 31) && 2 * (b_rows + 64) * p.ldb < (1ll << 31);
}
namespace {
template <int FMT, bool KCA, bool KCB>
hipError_t launch_ksplit16_kernel(const Gemm16Args& p, hipStream_t s, int tiles_m, int tiles_n, int group_m,
                                  unsigned blocks) {
    hipLaunchKernelGGL((gemm16_ksplit_kernel<FMT, KCA, KCB>), dim3(blocks), dim3(256), 0, s, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}
}  // namespace

// format: 0 bfloat16, 1 binary16; op_a / op_b: 1 if that factor is stored
// transposed.  64 x 64 tiles, tile-row groups of 8.
hipError_t launch_ksplit16(const Gemm16Args& p, hipStream_t s, int format, int op_a, int op_b) {
    const int tiles_m = ceil_div(p.M, 64), tiles_n = ceil_div(p.N, 64);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned nb = (unsigned)blocks;
    switch (4 * (format ? 1 : 0) + 2 * (op_a ? 1 : 0) + (op_b ? 1 : 0)) {
        case 0: return launch_ksplit16_kernel<0, true, false>(p, s, tiles_m, tiles_n, 8, nb);
        case 1: return launch_ksplit16_kernel<0, true, true>(p, s, tiles_m, tiles_n, 8, nb);
        case 2: return launch_ksplit16_kernel<0, false, false>(p, s, tiles_m, tiles_n, 8, nb);
        case 3: return launch_ksplit16_kernel<0, false, true>(p, s, tiles_m, tiles_n, 8, nb);
        case 4: return launch_ksplit16_kernel<1, true, false>(p, s, tiles_m, tiles_n, 8, nb);
        case 5: return launch_ksplit16_kernel<1, true, true>(p, s, tiles_m, tiles_n, 8, nb);
        case 6: return launch_ksplit16_kernel<1, false, false>(p, s, tiles_m, tiles_n, 8, nb);
        default: return launch_ksplit16_kernel<1, false, true>(p, s, tiles_m, tiles_n, 8, nb);
    }
}


}  // namespace gemmf32
