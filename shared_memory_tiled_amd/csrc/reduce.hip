// reduce.hip -- sum reduction, *out = x_0 + ... + x_{n-1}.
//
// The first page's "Reduction" section builds a block reduction in shared
// memory and improves it step by step; its multi-pass scheme reduces each
// block of values to one partial and runs again on the partials until one
// value is left.  Versions, adapted to gfx950's 64-lane waves:
//   0 interleaved     tree in LDS; at each level the thread owning the
//                     left slot of a pair adds (a remainder test picks one
//                     thread in 2, 4, 8, ..., scattered over every wave)
//   1 sequential      tree in LDS; the lowest-numbered threads add (adders
//                     packed at the front, whole waves idle, no remainder)
//   2 wave_shuffle    version 1 until one wave holds the data, then the wave
//                     folds it in registers with lane shuffles (no LDS
//                     round trips, no block barriers for the last 6 steps)
//   3 atomic          version 2 per block, then one float atomic add per
//                     block into *out (single pass; the order of the adds
//                     varies from run to run, so the last bits can too)
//   4 grid_vec        gfx950 layout: a fixed grid of 2048 blocks walks the
//                     array with nontemporal 128-bit loads (streamed data
//                     that is read once) into four accumulators per thread,
//                     folds waves by shuffles and blocks through LDS, and a
//                     second one-block launch folds the 2048 partials
//                     (deterministic; bound by HBM reads)
// Versions 0-2 and 4 write partials to a workspace: the caller's, or, for
// callers that cannot allocate, a fixed array in device memory (below);
// every version is deterministic except 3.
#include "launch.h"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace gemmf32 {

namespace {

constexpr int kBlock = 256;          // threads per block, values per block (versions 0-3)
constexpr int kGridBlocks = 2048;    // version 4: blocks of the first pass

// One wave's 64 values folded into lane 0 by shuffles (offsets 32 .. 1).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
    return v;
}

// The block's tree (versions 0-2).  Level j (j = 0, 1, ...) halves the
// number of live slots: each of its kBlock >> (j + 1) additions folds one
// slot into another.  The versions differ only in which thread performs
// which addition, which decides how the adding threads spread over waves.
//
// Interleaved pairs: a live slot at level j is a multiple of 2^j and
// absorbs the slot 2^j above it; each thread works on its own slot, so the
// adders are the threads whose index leaves no remainder modulo 2^(j+1) --
// one in every 2^(j+1), scattered through every wave until the tree is a
// wave wide.
struct InterleavedPairs {
    __device__ static bool adds(int t, int level) { return t % (2 << level) == 0; }
    __device__ static int partner(int t, int level) { return t + (1 << level); }
};
// Sequential pairs: at level j the live slots are the first kBlock >> j, and
// thread t folds slot t + (kBlock >> (j + 1)) into slot t, so the adders are
// the lowest-numbered threads and whole waves drop out as the tree narrows.
struct SequentialPairs {
    __device__ static int half(int level) { return kBlock >> (level + 1); }
    __device__ static bool adds(int t, int level) { return t < half(level); }
    __device__ static int partner(int t, int level) { return t + half(level); }
};

// Levels 0 .. LEVELS - 1 of the tree over `slots`, one block barrier after
// each so the next level reads finished sums.
template <class Pairs, int LEVELS>
__device__ __forceinline__ void fold_levels(float* slots, int t) {
    for (int level = 0; level < LEVELS; ++level) {
        if (Pairs::adds(t, level)) slots[t] += slots[Pairs::partner(t, level)];
        __syncthreads();
    }
}

constexpr int kLevels = 8;                 // log2(kBlock)
static_assert((1 << kLevels) == kBlock, "tree depth");

// Versions 0-3: block b folds values [256 b, 256 b + 256) of `in` (missing
// values count as +0) into part[b], or adds it to *out (version 3).
// Versions 0 and 1 run the whole tree in LDS; 2 and 3 run it until one wave
// holds the live slots (two levels), then fold that wave in registers.
template <int VERSION>
__global__ __launch_bounds__(kBlock) void reduce_block_kernel(int64_t n, const float* in, float* part) {
    __shared__ float slots[kBlock];
    const int t = threadIdx.x;
    const int64_t i = (int64_t)blockIdx.x * kBlock + t;
    slots[t] = i < n ? in[i] : 0.0f;
    __syncthreads();
    if constexpr (VERSION <= 1) {
        using Pairs = std::conditional_t<VERSION == 0, InterleavedPairs, SequentialPairs>;
        fold_levels<Pairs, kLevels>(slots, t);
        if (t == 0) part[blockIdx.x] = slots[0];
    } else {
        fold_levels<SequentialPairs, 2>(slots, t);        // 256 -> 64 live slots
        if (t < 64) {                                     // wave 0, wave-uniform branch
            const float v = wave_sum(slots[t]);
            if (t == 0) {
                if constexpr (VERSION == 2) part[blockIdx.x] = v;
                else atomicAdd(part, v);                  // part is *out for version 3
            }
        }
    }
}

__global__ void zero_one_kernel(float* out) { *out = 0.0f; }

// Four floats at 4-byte alignment (a dword-aligned 128-bit load is legal on
// gfx9, which runs global memory in unaligned mode).
typedef float floatx4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Version 4, first pass: a grid-stride walk over 16-byte chunks.
__global__ __launch_bounds__(kBlock) void reduce_grid_vec_kernel(int64_t n, const float* in, float* part) {
    __shared__ float wave_part[kBlock / 64];
    const int tid = threadIdx.x;
    const int64_t chunks = n / 4;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    for (int64_t c = (int64_t)blockIdx.x * kBlock + tid; c < chunks; c += stride) {
        const floatx4_a4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4_a4*>(in + 4 * c));
        a0 += v[0];
        a1 += v[1];
        a2 += v[2];
        a3 += v[3];
    }
    // the last n % 4 values go to the first threads of block 0
    if (blockIdx.x == 0 && tid < (int)(n % 4)) a0 += in[4 * chunks + tid];
    float v = wave_sum((a0 + a1) + (a2 + a3));
    if ((tid & 63) == 0) wave_part[tid >> 6] = v;
    __syncthreads();
    if (tid == 0) part[blockIdx.x] = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
}

// Version 4, second pass: one block folds `count` partials.
__global__ __launch_bounds__(kBlock) void reduce_final_kernel(int count, const float* part, float* out) {
    __shared__ float wave_part[kBlock / 64];
    const int tid = threadIdx.x;
    float a = 0.0f;
    for (int i = tid; i < count; i += kBlock) a += part[i];
    const float v = wave_sum(a);
    if ((tid & 63) == 0) wave_part[tid >> 6] = v;
    __syncthreads();
    if (tid == 0) *out = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int reduce_num_variants() { return 5; }

const char* reduce_variant_name(int v) {
    static const char* const names[] = {"interleaved", "sequential", "wave_shuffle", "atomic", "grid_vec"};
    return (v >= 0 && v < 5) ? names[v] : nullptr;
}

// Floats of workspace each version needs for n values.
int64_t reduce_workspace_floats(int variant, int64_t n) {
    if (variant == 3 || n < 1) return 0;
    if (variant == 4) return kGridBlocks;
    int64_t total = 0;                 // partials of every pass but the last
    for (int64_t m = ceil_div64(n, kBlock); m > 1; m = ceil_div64(m, kBlock)) total += m;
    return total;
}

hipError_t launch_reduce(int variant, int64_t n, const float* x, float* out, float* ws, hipStream_t s) {
    if (n == 0) {
        hipLaunchKernelGGL(zero_one_kernel, dim3(1), dim3(1), 0, s, out);
        return hipGetLastError();
    }
    if (variant == 4) {
        const int64_t need = ceil_div64(ceil_div64(n, 4), kBlock);
        const int blocks = (int)(need < kGridBlocks ? need : kGridBlocks);
        hipLaunchKernelGGL(reduce_grid_vec_kernel, dim3(blocks), dim3(kBlock), 0, s, n, x, ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kBlock), 0, s, blocks, ws, out);
        return hipGetLastError();
    }
    if (variant == 3) {
        const int64_t blocks = ceil_div64(n, kBlock);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(zero_one_kernel, dim3(1), dim3(1), 0, s, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(reduce_block_kernel<3>, dim3((unsigned)blocks), dim3(kBlock), 0, s, n, x, out);
        return hipGetLastError();
    }
    // Multi-pass: each pass turns m values into ceil(m / 256) partials; the
    // partials of successive passes sit one after another in the workspace,
    // and the last pass writes *out.
    const float* src = x;
    float* dst = ws;
    int64_t m = n;
    while (true) {
        const int64_t blocks = ceil_div64(m, kBlock);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        float* target = blocks == 1 ? out : dst;
        const dim3 grid((unsigned)blocks), block(kBlock);
        switch (variant) {
            case 0: hipLaunchKernelGGL(reduce_block_kernel<0>, grid, block, 0, s, m, src, target); break;
            case 1: hipLaunchKernelGGL(reduce_block_kernel<1>, grid, block, 0, s, m, src, target); break;
            default: hipLaunchKernelGGL(reduce_block_kernel<2>, grid, block, 0, s, m, src, target); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || blocks == 1) return e;
        src = dst;
        dst += blocks;
        m = blocks;
    }
}

// ------------------------------------------------------------ fixed scratch
//
// For callers that cannot allocate device memory (code under stream capture,
// loops that must not call the allocator): the partials go to this array,
// which every GPU the library runs on holds for the life of the process.
// Each device has its own copy at its own address; on the host the name
// `scratch` is only a symbol, so kernels receive the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.  Every call on one GPU shares that GPU's copy: calls that
// overlap on one GPU (two streams, two host threads) race.  Nothing in it
// needs clearing: every version writes each partial before reading it.
__device__ __align__(256) float scratch[kReduceScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t reduce_scratch(int device, float** ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    float* p = g_scratch[device].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[device].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (addr == nullptr) return hipErrorInvalidSymbol;
            p = static_cast<float*>(addr);
            g_scratch[device].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace gemmf32
