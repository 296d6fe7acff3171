// probe.hip -- a measurement helper, not part of the product: loops of
// non-packed binary32 fused multiply-adds on the vector ALU, timed by the
// caller, that give the issue rate of the register-blocked rung's
// instruction (v_fmac_f32) on gfx950.  Three operand forms:
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

}  // namespace

hipError_t launch_valu_probe(int form, int blocks, int iters, float* out, uint64_t* stamps, hipStream_t s) {
    switch (form) {
        case 0: hipLaunchKernelGGL(valu_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
        case 1: hipLaunchKernelGGL(valu_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
        default: hipLaunchKernelGGL(valu_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, out, stamps, iters, 0.999f); break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
