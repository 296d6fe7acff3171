// probe.hip -- measurement helpers, not part of the product.
//
// 1. Loops of non-packed binary32 fused multiply-adds on the vector ALU,
// timed by the caller, that give the issue rate of the register-blocked
// rung's instruction (v_fmac_f32) on gfx950.  Three operand forms:
//   0  one operand in a scalar register (v_fmac_f32 acc, v_x, s_b)
//   1  all operands in vector registers (v_fmac_f32 acc, v_x, v_y), 16
//      independent accumulators per lane
//   2  the register-blocked rung's inner step: an 8 x 8 outer product of
//      vector registers into 64 accumulators per lane
// Every lane of every wave does ITERS x 16 (forms 0, 1) or ITERS / 4 x 64
// (form 2) FMAs.  Lane 0 of each wave records the shader clock counter
// (s_memtime) and the fixed 100 MHz counter (s_memrealtime) before and after
// its loop, so the caller can state the clock the loop ran at.
#include "launch.h"

namespace gemmf32 {

namespace {

__device__ __forceinline__ void stamp(uint64_t* t, int slot) {
    const uint64_t c = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
        const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
        t[4 * wave + 2 * slot] = c;
        t[4 * wave + 2 * slot + 1] = r;
    }
}

template <int FORM>
__global__ __launch_bounds__(256) void valu_probe_kernel(float* out, uint64_t* t, int iters, float b) {
    stamp(t, 0);
    float s = 0.0f;
    if constexpr (FORM == 2) {
        float acc[64], x[8], y[8];
#pragma unroll
        for (int j = 0; j < 64; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = (threadIdx.x + j) * 1e-7f;
            y[j] = b + threadIdx.x * 1e-9f * j;
        }
        for (int i = 0; i < iters / 4; ++i) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[8 * u + v] = __builtin_fmaf(x[u], y[v], acc[8 * u + v]);
        }
#pragma unroll
        for (int j = 0; j < 64; ++j) s += acc[j];
    } else {
        float a[16], x[16], y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            a[j] = 0.0f;
            x[j] = (threadIdx.x + j) * 1e-7f;
            y[j] = b + threadIdx.x * 1e-9f * j;
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 16; ++j) a[j] = __builtin_fmaf(x[j], FORM == 0 ? b : y[j], a[j]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) s += a[j];
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    stamp(t, 1);
}

// 2. One wave reading LDS: lane l reads `width` bytes at byte offset
// offs[l] (masked into a 64 KB array and aligned to the width) `iters`
// times, each read waited for in the same instruction sequence; with the
// LDS bank-conflict counter per dispatch, a set of offsets tells which lanes
// one read cycle serves.  Forms: 0 ds_read_b32, 1 ds_read_b64, 2
// ds_read_b128, 3 ds_read_b64_tr_b16.
template <int FORM>
__global__ __launch_bounds__(64) void lds_probe_kernel(const int* __restrict__ offs, int iters,
                                                       unsigned* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) unsigned lds[16384];          // 64 KB
    const int t = threadIdx.x;
    for (int i = t; i < 16384; i += 64) lds[i] = (unsigned)i * 2654435761u;
    __syncthreads();
    constexpr uint32_t kMask = FORM == 0 ? 0xFFFCu : FORM == 2 ? 0xFFF0u : 0xFFF8u;
    const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds +
                          ((uint32_t)offs[t] & kMask);
    unsigned acc = 0;
    for (int i = 0; i < iters; ++i) {
        if constexpr (FORM == 0) {
            unsigned v;
            asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
            acc += v;
        } else if constexpr (FORM == 2) {
            typedef unsigned u4 __attribute__((ext_vector_type(4)));
            u4 v;
            asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
            acc += v[0] ^ v[1] ^ v[2] ^ v[3];
        } else {
            typedef unsigned u2 __attribute__((ext_vector_type(2)));
            u2 v;
            if constexpr (FORM == 1)
                asm volatile("ds_read_b64 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
            else
                asm volatile("ds_read_b64_tr_b16 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
            acc += v[0] ^ v[1];
        }
    }
    out[t] = acc;
}

}  // namespace

hipError_t launch_lds_probe(int form, const int* offs, int iters, unsigned* out, hipStream_t s) {
    switch (form) {
        case 0: hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(1), dim3(64), 0, s, offs, iters, out); break;
        case 1: hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(1), dim3(64), 0, s, offs, iters, out); break;
        case 2: hipLaunchKernelGGL(lds_probe_kernel<2>, dim3(1), dim3(64), 0, s, offs, iters, out); break;
        default: hipLaunchKernelGGL(lds_probe_kernel<3>, dim3(1), dim3(64), 0, s, offs, iters, out); break;
    }
    return hipGetLastError();
}

hipError_t launch_valu_probe(int form, int blocks, int iters, float* out, uint64_t* stamps, hipStream_t s) {
    switch (form) {
        case 0: hipLaunchKernelGGL(valu_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
        case 1: hipLaunchKernelGGL(valu_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
        default: hipLaunchKernelGGL(valu_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
