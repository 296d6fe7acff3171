// transpose.hip -- the shared-tile matrix transpose, out[c][r] = in[r][c].
//
// The first page's "Bank Conflict" section transposes through a shared tile:
// a block reads a tile of `in` row by row (coalesced), and writes it to
// `out` row by row too, reading the tile by columns.  The column read is
// where banks collide: a [32][32] tile puts a whole column in one bank (the
// page's 32-way conflict on 32 banks), a [32][33] tile shifts each row by one
// bank, and the XOR swizzle tile[y][x ^ y] spreads rows and columns alike.
//
// Variants:
//   0 naive          no LDS: each thread reads one element (coalesced) and
//                    writes it transposed (lanes 4 * ld_out bytes apart)
//   1 tile32         the page's kernel: [32][32] tile, 32 x 32 threads
//   2 tile32_pad     [32][33] tile
//   3 tile32_swizzle [32][32] tile indexed [y][x ^ y]
//   4 tile64_vec     gfx950 layout: 64 x 64 tile, 256 threads, 128-bit global
//                    and LDS accesses only; each thread transposes a 4 x 4
//                    block in registers, and the 16-byte chunks of each LDS
//                    row are permuted by an XOR so stores and reads are
//                    conflict free on gfx950's LDS (see the kernel).
//   5 tile128_vec    the same with a 128 x 128 tile (512-byte row segments)
//   6 tile64_vec_diag  tile64_vec with tiles handed out in diagonal order
//   7 tile64_vec_diag_nt, 8 tile64_vec_nt  variants 6 and 4 with nontemporal
//                    global loads and stores (for arrays larger than the last
//                    level cache, where every byte is moved once anyway)
// Every variant guards each element against the matrix edges; nothing is
// read or written outside `rows x cols` (in) and `cols x rows` (out).
#include "launch.h"

namespace gemmf32 {

namespace {

__global__ __launch_bounds__(256) void transpose_naive_kernel(int rows, int cols, const float* in,
                                                              int64_t ld_in, float* out,
                                                              int64_t ld_out, int tiles_c) {
    // 64 x 64 tile per block of 64 x 4 threads, 16 rows per thread
    const int r0 = (int)(blockIdx.x / tiles_c) * 64, c0 = (int)(blockIdx.x % tiles_c) * 64;
    const int c = c0 + (int)threadIdx.x;
    if (c >= cols) return;                      // no barrier in this kernel
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + (int)threadIdx.y + 4 * i;
        if (r < rows) out[(int64_t)c * ld_out + r] = in[(int64_t)r * ld_in + c];
    }
}

// The page's kernel with a [32][32 + PAD] tile, or the XOR-swizzled [32][32]
// tile.  One element per thread, 32 x 32 threads.
template <int PAD, bool SWIZZLE>
__global__ __launch_bounds__(1024) void transpose_tile32_kernel(int rows, int cols, const float* in,
                                                                int64_t ld_in, float* out,
                                                                int64_t ld_out, int tiles_c) {
    constexpr int S = 32 + PAD;
    __shared__ float tile[32 * S];
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int r0 = (int)(blockIdx.x / tiles_c) * 32, c0 = (int)(blockIdx.x % tiles_c) * 32;
    // row-wise write of the tile: element (ty, tx) of the input tile
    if (r0 + ty < rows && c0 + tx < cols)
        tile[ty * S + (SWIZZLE ? (tx ^ ty) : tx)] = in[(int64_t)(r0 + ty) * ld_in + c0 + tx];
    __syncthreads();
    // column-wise read: output row c0 + ty holds input column c0 + ty
    if (c0 + ty < cols && r0 + tx < rows)
        out[(int64_t)(c0 + ty) * ld_out + r0 + tx] = tile[tx * S + (SWIZZLE ? (ty ^ tx) : ty)];
}

// T x T tile, 256 threads, every LDS access 128 bits wide.  A thread owns 4 x
// 4 blocks of input rows 4i .. 4i+3 and columns 4j .. 4j+3: four 128-bit row
// loads, a transpose in registers, and four 128-bit LDS stores into the
// transposed tile, whose row c is output row c0 + c (input column).  The
// 16-byte chunk k of LDS row c sits at chunk position k ^ (c/4 % 8): the
// eight lanes one 128-bit store serves per cycle (32 banks; consecutive
// lanes hold consecutive j) then write eight different bank groups, and the
// sixteen lanes one 128-bit read serves (64 banks) read sixteen.  Scalar LDS stores would
// not do: the compiler pairs them into one instruction whose two words sit
// 64 words apart, in the same bank.
template <int T>
__device__ __forceinline__ int tvec_word(int c, int chunk) {
    return c * T + 4 * (chunk ^ ((c >> 2) & 7));
}

// Four floats at 4-byte alignment (a dword-aligned 128-bit access is legal on
// gfx9, which runs global memory in unaligned mode).
typedef float floatx4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// T x T tile (T = 64 or 128), 256 threads; each thread transposes
// (T/4)^2 / 256 blocks of 4 x 4.  NT: nontemporal global loads and stores;
// NTS: nontemporal stores only (the loads keep the input cacheable).
template <int T, bool DIAGONAL, bool NT, bool NTS = NT>
__global__ __launch_bounds__(256) void transpose_tile_vec_kernel(int rows, int cols, const float* in,
                                                                 int64_t ld_in, float* out,
                                                                 int64_t ld_out, int tiles_c) {
    constexpr int NB = T / 4;                 // 4 x 4 blocks (and 16-byte chunks) per tile edge
    constexpr int PER = NB * NB / 256;
    static_assert(PER * 256 == NB * NB && NB >= 16, "tile shape");
    __shared__ __attribute__((aligned(16))) float tile[T * T];
    const int tid = threadIdx.x;
    int tr = (int)(blockIdx.x / tiles_c), tc = (int)(blockIdx.x % tiles_c);
    if (DIAGONAL) {
        // Diagonal order: blocks that run at the same time take tiles from
        // different tile rows AND columns, so their input rows and output
        // rows (ld apart) do not all start at one offset modulo a large
        // power of two.  Only full tile grids are reordered (a bijection of
        // the tiles_r x tiles_c grid when it is square).
        const int tiles_r = (int)(gridDim.x / tiles_c);
        if (tiles_r == tiles_c) {
            tr = (int)blockIdx.x % tiles_r;
            tc = ((int)blockIdx.x / tiles_r + tr) % tiles_c;
        }
    }
    const int r0 = tr * T, c0 = tc * T;
    const bool inside = r0 + T <= rows && c0 + T <= cols;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int b = tid + 256 * p;
        const int i = b / NB, j = b % NB;       // input rows 4i .. 4i+3, columns 4j .. 4j+3
        floatx4 v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * i + e;
            const float* src = in + (int64_t)(r0 + r) * ld_in + c0 + 4 * j;
            if (inside && NT) v[e] = __builtin_nontemporal_load(reinterpret_cast<const floatx4_a4*>(src));
            else if (inside) __builtin_memcpy(&v[e], src, 16);
            else v[e] = load4_ghost(in, r0 + r, rows, c0 + 4 * j, cols, ld_in);   // zeros never reach out
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // column 4j + e of the block = output row 4j + e
            const floatx4 t = {v[0][e], v[1][e], v[2][e], v[3][e]};
            *reinterpret_cast<floatx4*>(&tile[tvec_word<T>(4 * j + e, i)]) = t;
        }
    }
    __syncthreads();
    // write: chunk q is output row q / NB (input column), input rows 4 (q % NB) .. +3
#pragma unroll
    for (int u = 0; u < T * T / 1024; ++u) {
        const int q = tid + 256 * u;
        const int c = q / NB, k = q % NB;
        const floatx4 w = *reinterpret_cast<const floatx4*>(&tile[tvec_word<T>(c, k)]);
        float* dst = out + (int64_t)(c0 + c) * ld_out + r0 + 4 * k;
        if (inside && NTS) __builtin_nontemporal_store(floatx4_a4(w), reinterpret_cast<floatx4_a4*>(dst));
        else if (inside) __builtin_memcpy(dst, &w, 16);
        else store4_guarded(out, c0 + c, cols, r0 + 4 * k, rows, ld_out, w);
    }
}

}  // namespace

int transpose_num_variants() { return 11; }

const char* transpose_variant_name(int v) {
    static const char* const names[] = {"naive",           "tile32",         "tile32_pad",
                                        "tile32_swizzle",  "tile64_vec",     "tile128_vec",
                                        "tile64_vec_diag", "tile64_vec_diag_nt", "tile64_vec_nt",
                                        "tile64_vec_diag_ntstore", "tile128_vec_diag_ntstore"};
    return (v >= 0 && v < 11) ? names[v] : nullptr;
}

hipError_t launch_transpose(int variant, int rows, int cols, const float* in, int64_t ld_in,
                            float* out, int64_t ld_out, hipStream_t s) {
    const int tile = (variant >= 1 && variant <= 3) ? 32 : ((variant == 5 || variant == 10) ? 128 : 64);
    const int tiles_c = ceil_div(cols, tile);
    const int64_t blocks = (int64_t)tiles_c * ceil_div(rows, tile);
    const int64_t threads = (variant >= 1 && variant <= 3) ? 1024 : 256;
    if (blocks * threads > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (variant) {
        case 0:
            hipLaunchKernelGGL(transpose_naive_kernel, grid, dim3(64, 4), 0, s, rows, cols, in, ld_in,
                               out, ld_out, tiles_c);
            break;
        case 1:
            hipLaunchKernelGGL((transpose_tile32_kernel<0, false>), grid, dim3(32, 32), 0, s, rows, cols,
                               in, ld_in, out, ld_out, tiles_c);
            break;
        case 2:
            hipLaunchKernelGGL((transpose_tile32_kernel<1, false>), grid, dim3(32, 32), 0, s, rows, cols,
                               in, ld_in, out, ld_out, tiles_c);
            break;
        case 3:
            hipLaunchKernelGGL((transpose_tile32_kernel<0, true>), grid, dim3(32, 32), 0, s, rows, cols,
                               in, ld_in, out, ld_out, tiles_c);
            break;
        case 5:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<128, false, false>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        case 6:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<64, true, false>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        case 7:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<64, true, true>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        case 8:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<64, false, true>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        case 9:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<64, true, false, true>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        case 10:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<128, true, false, true>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
        default:
            hipLaunchKernelGGL((transpose_tile_vec_kernel<64, false, false>), grid, dim3(256), 0, s, rows,
                               cols, in, ld_in, out, ld_out, tiles_c);
            break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
