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

// 3. The rate of 1 KB wave copies from an L2-resident buffer per CU: each
// block (4 waves) reads its own 64 KB window of src, wave w the 16 KB at
// 16 KB w, in 1 KB wave loads (16 bytes a lane) cycling through the 16 KB,
// keeping 8 to 16 loads in flight; mode 0 loads into LDS
// (buffer_load_dwordx4 ... lds, as the 16-bit kernels' copies), mode 1 into
// vector registers (the loads of one group of eight are consumed while the
// next group is in flight).  Lane 0 of each wave records the shader clock
// counter around its loop.
template <int MODE>
__global__ __launch_bounds__(256) void copy_probe_kernel(const unsigned* __restrict__ src, int iters,
                                                         unsigned* __restrict__ out, uint64_t* __restrict__ cycles) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) unsigned char lds[32768];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned*>(src) + ((int64_t)blockIdx.x * 65536 + (int64_t)w * 16384) / 4, (short)0, 16384,
        0x00020000);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    u4 acc = {0, 0, 0, 0}, v0[8], v1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v0[j] = v1[j] = u4{0, 0, 0, 0};
    for (int i = 0; i < iters; i += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u4 (&cur)[8] = h ? v1 : v0;
            u4 (&prev)[8] = h ? v0 : v1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int voff = ((i * 3 + h * 8 + j) % 16) * 1024 + 16 * lane;      // below 16384
                if constexpr (MODE == 0) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rs, (__attribute__((address_space(3))) void*)(lds + (w * 8 + j) * 1024), 16, voff, 0, 0, 0);
                } else {
                    cur[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
                }
            }
            if constexpr (MODE == 0) {
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc ^= prev[j];
            }
        }
    }
    if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v1[j];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    __syncthreads();
    out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ lds[threadIdx.x * 16];
    if (lane == 0) cycles[blockIdx.x * 4 + w] = t1 - t0;
}

}  // namespace

hipError_t launch_copy_probe(int mode, int blocks, const unsigned* src, int iters, unsigned* out, uint64_t* cycles,
                             hipStream_t s) {
    if (mode == 0) hipLaunchKernelGGL(copy_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, src, iters, out, cycles);
    else hipLaunchKernelGGL(copy_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, src, iters, out, cycles);
    return hipGetLastError();
}

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
