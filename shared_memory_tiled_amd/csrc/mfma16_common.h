// mfma16_common.h -- device helpers shared by the 16-bit (bfloat16 /
// binary16) kernels: vector types, LDS reads (plain and transposed), waits
// tied to the registers they complete, and compile-time unrolling (not part
// of the public interface).
#pragma once

#include "launch.h"

#include <type_traits>
#include <utility>

namespace gemmf32 {

namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// Four 16-bit values through ds_read_b64_tr_b16.  Within each group of 16
// lanes, value e of lane i is element i % 4 of the 8 bytes addressed by lane
// 4 e + i / 4.  So if lane j of a group addresses row kb + j / 4, columns
// nb + 4 (j % 4) .. +3 of a row-major tile, lane i receives the column
// nb + i, rows kb .. kb + 3: four consecutive k of one n.
//
// Issued as inline assembly: the compiler would otherwise wait for every
// outstanding global -> LDS copy before the first such read (it cannot tell
// that the copies fill the other stage).  The "memory" clobber keeps the
// reads in order with the barriers; wait_tied() below is their wait.
__device__ __forceinline__ u32x2 read_tr16(uint32_t lds_byte_addr) {
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(lds_byte_addr) : "memory");
    return v;
}

// Waits for all outstanding LDS reads; the fragments pass through the wait
// as operands, so no use of them can be scheduled before it.
template <int N>
__device__ __forceinline__ void wait_tied(u32x4 (&b)[N]) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 5 || N == 6 || N == 8, "fragment count");
    if constexpr (N == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b[0]) : : "memory");
    if constexpr (N == 2) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b[0]), "+v"(b[1]) : : "memory");
    if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]) : : "memory");
    if constexpr (N == 5)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4])
                     :
                     : "memory");
    if constexpr (N == 6)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5])
                     :
                     : "memory");
    if constexpr (N == 8)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7])
                     :
                     : "memory");
}

// The same for fragments held as 64-bit halves (two transposed reads each).
__device__ __forceinline__ void wait_tied(u32x2 (&h)[8][2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(h[0][0]), "+v"(h[0][1]), "+v"(h[1][0]), "+v"(h[1][1]), "+v"(h[2][0]), "+v"(h[2][1]),
                   "+v"(h[3][0]), "+v"(h[3][1]), "+v"(h[4][0]), "+v"(h[4][1]), "+v"(h[5][0]), "+v"(h[5][1]),
                   "+v"(h[6][0]), "+v"(h[6][1]), "+v"(h[7][0]), "+v"(h[7][1])
                 :
                 : "memory");
}

__device__ __forceinline__ void wait_tied(u32x2 (&h)[5][2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(h[0][0]), "+v"(h[0][1]), "+v"(h[1][0]), "+v"(h[1][1]), "+v"(h[2][0]), "+v"(h[2][1]),
                   "+v"(h[3][0]), "+v"(h[3][1]), "+v"(h[4][0]), "+v"(h[4][1])
                 :
                 : "memory");
}

__device__ __forceinline__ void wait_tied(u32x2 (&h)[6][2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(h[0][0]), "+v"(h[0][1]), "+v"(h[1][0]), "+v"(h[1][1]), "+v"(h[2][0]), "+v"(h[2][1]),
                   "+v"(h[3][0]), "+v"(h[3][1]), "+v"(h[4][0]), "+v"(h[4][1]), "+v"(h[5][0]), "+v"(h[5][1])
                 :
                 : "memory");
}

// Keeps fragments alive up to this point (no register of theirs is handed
// to another value before it).
template <int N>
__device__ __forceinline__ void keep_alive(const u32x4 (&b)[N]) {
    static_assert(N == 8, "fragment count");
    asm volatile("" ::"v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]));
}
__device__ __forceinline__ void keep_alive(const u32x2 (&h)[8][2]) {
    asm volatile("" ::"v"(h[0][0]), "v"(h[0][1]), "v"(h[1][0]), "v"(h[1][1]), "v"(h[2][0]), "v"(h[2][1]),
                 "v"(h[3][0]), "v"(h[3][1]), "v"(h[4][0]), "v"(h[4][1]), "v"(h[5][0]), "v"(h[5][1]), "v"(h[6][0]),
                 "v"(h[6][1]), "v"(h[7][0]), "v"(h[7][1]));
}

// Byte address inside LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes of LDS at a byte address.
__device__ __forceinline__ u32x4 lds_read128(uint32_t lds_byte_addr) {
    typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
    return *(lds_u32x4*)(uintptr_t)lds_byte_addr;
}

// read_tr16 with a compile-time byte offset in the instruction.
__device__ __forceinline__ u32x2 read_tr16_off(uint32_t lds_byte_addr, int off) {
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_byte_addr), "i"(off) : "memory");
    return v;
}

// D = A B + C on one 16 x 16 x 32 block (format 0 bfloat16, 1 binary16):
// lane l supplies A[l % 16][8 (l / 16) .. + 7] and B[8 (l / 16) .. + 7][l %
// 16]; accumulator register r holds D[4 (l / 16) + r][l % 16].
template <int FMT>
__device__ __forceinline__ floatx4 mfma16x16(u32x4 a, u32x4 b, floatx4 c) {
    if constexpr (FMT == 0)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c,
                                                      0, 0, 0);
}

template <typename F, int... Q>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Q...>) {
    (f(std::integral_constant<int, Q>{}), ...);
}
// f(std::integral_constant<int, q>{}) for q = 0 .. N - 1, in order: every
// index is a compile-time constant, so arrays indexed by it stay in registers
// (a loop under #pragma unroll is unrolled only after the pass that would
// have kept them there).
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    unroll_seq(f, std::make_integer_sequence<int, N>{});
}

}  // namespace

}  // namespace gemmf32
