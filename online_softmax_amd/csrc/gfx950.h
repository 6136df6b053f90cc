// Device building blocks shared by the attention kernels for gfx950: vector
// types, the 32x32x16 matrix product of 16-bit fragments, packing to 16-bit
// with round-to-nearest-even, half-wave reductions, the direct
// global-to-LDS load through a buffer resource, and load-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef uint32_t v4u32 __attribute__((__vector_size__(16)));
typedef uint32_t v2u32 __attribute__((__vector_size__(8)));
typedef float v4f32 __attribute__((__vector_size__(16)));
typedef float v16f32 __attribute__((__vector_size__(64)));
typedef __bf16 v8bf16 __attribute__((__vector_size__(16)));
typedef _Float16 v8f16 __attribute__((__vector_size__(16)));
typedef __bf16 v2bf16 __attribute__((__vector_size__(4)));
typedef _Float16 v2f16 __attribute__((__vector_size__(4)));

constexpr float kLn2 = 0.693147180559945309417f;

// One 32x32x16 product of 16-bit fragments (4 dwords per lane each).
template <int DT>
__device__ inline v16f32 mfma16(v4u32 a, v4u32 b, v16f32 c);
template <>
__device__ inline v16f32 mfma16<ATTN_DT_BF16>(v4u32 a, v4u32 b, v16f32 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(v8bf16, a), __builtin_bit_cast(v8bf16, b), c, 0, 0,
        0);
}
template <>
__device__ inline v16f32 mfma16<ATTN_DT_F16>(v4u32 a, v4u32 b, v16f32 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(v8f16, a), __builtin_bit_cast(v8f16, b), c, 0, 0, 0);
}

// Two floats -> one dword of two 16-bit values, round to nearest even; the
// first argument lands in the low half (the lower address).
template <int DT>
__device__ inline uint32_t pack2(float a, float b);
template <>
__device__ inline uint32_t pack2<ATTN_DT_BF16>(float a, float b) {
    v2bf16 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}
template <>
__device__ inline uint32_t pack2<ATTN_DT_F16>(float a, float b) {
    v2f16 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// max / sum of x over lanes l and l ^ 32 (the two halves holding one query).
__device__ inline float halves_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
                 __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ inline float halves_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) +
           __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The 16-bit value in the low / high half of a dword, widened to float.
template <int DT>
__device__ inline float lo16(uint32_t x);
template <int DT>
__device__ inline float hi16(uint32_t x);
template <>
__device__ inline float lo16<ATTN_DT_BF16>(uint32_t x) {
    return __builtin_bit_cast(float, x << 16);
}
template <>
__device__ inline float hi16<ATTN_DT_BF16>(uint32_t x) {
    return __builtin_bit_cast(float, x & 0xffff0000u);
}
template <>
__device__ inline float lo16<ATTN_DT_F16>(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}
template <>
__device__ inline float hi16<ATTN_DT_F16>(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// Sum of the two 16-bit values packed in `pair`, added to acc in fp32
// (v_dot2c_f32_{bf16,f16} against (1, 1)): the row sum of the rounded p.
template <int DT>
__device__ inline float sum2(uint32_t pair, float acc);
template <>
__device__ inline float sum2<ATTN_DT_BF16>(uint32_t pair, float acc) {
    const v2bf16 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf16, pair), one,
                                           acc, false);
}
template <>
__device__ inline float sum2<ATTN_DT_F16>(uint32_t pair, float acc) {
    const v2f16 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2f16, pair), one, acc,
                                  false);
}

typedef short v4i16 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) void lds_void;

typedef uint32_t v4u32_rsrc __attribute__((__vector_size__(16)));

// Buffer resource over `bytes` bytes from `base` (raw, dword data format),
// built from wave-uniform values so it lives in scalar registers.
__device__ inline v4u32_rsrc buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    v4u32_rsrc r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// One direct load of 16 bytes per lane from buffer `rsrc` into LDS
// (buffer_load_dwordx4 ... lds): lane l fetches bytes soff + voff[l] of the
// buffer and they land at LDS byte offset lds_off + 16 * l (lds_off and soff
// wave-uniform). The buffer form is used because, measured on gfx950, its
// issue is delayed far less than the flat/global form's while the other
// wave on the SIMD runs matrix instructions. Issued as inline assembly so the
// compiler does not treat the LDS write as aliasing every later LDS read and
// drain the load queue before each tile; completion is tracked explicitly
// with wait_vmcnt and a barrier. A load that takes its LDS address from M0
// needs one wait state after the scalar write of M0, hence the s_nop.
__device__ inline void dma16(v4u32_rsrc rsrc, uint32_t voff, uint32_t soff,
                             uint32_t lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// Wait until at most n of this wave's vector-memory operations are pending
// (other counters untouched).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until every LDS (and scalar memory) operation of this wave has
// completed (vector-memory and export counters untouched).
__device__ inline void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Wait until at most `in_flight` (0, 2, 4, 6 or 8: whole load batches) of
// this wave's loads are pending.
__device__ inline void wait_loads(int in_flight) {
    if (in_flight >= 8)
        wait_vmcnt<8>();
    else if (in_flight >= 6)
        wait_vmcnt<6>();
    else if (in_flight >= 4)
        wait_vmcnt<4>();
    else if (in_flight >= 2)
        wait_vmcnt<2>();
    else
        wait_vmcnt<0>();
}

}  // namespace attn
