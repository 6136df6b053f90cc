// Tile helpers shared by the backward kernels: direct loads of 64-row
// tiles into LDS in the swz_b swizzle (fused_layout.h), row and transposed
// fragment reads from such tiles, and the store of 32 rows held transposed in
// two accumulators.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fused_layout.h"
#include "gfx950.h"

namespace attn {

// One direct load of 4 bytes per lane from buffer `rsrc` into LDS: lane l
// fetches bytes voff[l] and they land at lds_off + 4 * l.
__device__ inline void dma4(v4u32_rsrc rsrc, uint32_t voff, uint32_t lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_off), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// The two direct loads (2 wave instructions) of one 64-row tile of a slice
// buffer into `off`: rows from row0, rows past T clamped to T-1.
__device__ inline void load_btile(v4u32_rsrc rs, const uint32_t (&voff)[2], int row0, int T,
                                  int wave_u, uint32_t off) {
    if (row0 + 64 <= T) {
        const uint32_t soff = (uint32_t)row0 * (kHeadDim * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(rs, voff[i], soff, off + 1024 * (2 * wave_u + i));
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = min(row0 + (int)(voff[i] >> 7), T - 1);
            dma16(rs, (uint32_t)r * (kHeadDim * 2) + (voff[i] & 127), 0u,
                  off + 1024 * (2 * wave_u + i));
        }
    }
}

// Row fragments (A operand) of both 32-row halves of a tile at step ks.
__device__ inline v4u32 brow(const char* __restrict__ tile, uint32_t lane_base, int mt) {
    return *(const v4u32*)(tile + lane_base + kBfragMtStride * mt);
}
// Transposed fragment (A operand, columns 32ct..+31 as rows) at step ks.
__device__ inline v4u32 btr(const char* __restrict__ tile, uint32_t b0, uint32_t b1, int ks) {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const char* p0 = tile + b0 + kBtrKsStride * ks;
    const char* p1 = tile + b1 + kBtrKsStride * ks;
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
    const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
    const v2u32 x2 = __builtin_bit_cast(v2u32, x), y2 = __builtin_bit_cast(v2u32, y);
    return (v4u32){x2[0], x2[1], y2[0], y2[1]};
}

// A lane's fragment base in a tile whose ring stage is chosen at run time:
// the LDS byte address of tile + lane_base, kept opaque to the compiler so
// that the fragment reads from it take their constant parts (half, step) as
// instruction offsets. Left alone, the compiler folds those constants into
// one register per fragment outside the loop and adds the stage to every one
// of them on every tile. `tile` must be the same for every lane of the wave
// (a ring stage picked by the loop counter): its offset passes through a
// scalar register.
typedef __attribute__((address_space(3))) char lds_char;
__device__ inline const lds_char* lane_tile(const char* tile, uint32_t lane_base) {
    uint32_t t = (uint32_t)(uintptr_t)(lds_void*)tile;  // wave-uniform
    asm("" : "+s"(t));
    uint32_t a = t + lane_base;
    asm("" : "+v"(a));
    return (const lds_char*)(uintptr_t)a;
}
// brow and btr from such bases
__device__ inline v4u32 brow_at(const lds_char* p, int mt) {
    typedef __attribute__((address_space(3))) v4u32 lds_v4u32;
    return *(const lds_v4u32*)(p + kBfragMtStride * mt);
}
__device__ inline v4u32 btr_at(const lds_char* p0, const lds_char* p1, int ks) {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + kBtrKsStride * ks));
    const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1 + kBtrKsStride * ks));
    const v2u32 x2 = __builtin_bit_cast(v2u32, x), y2 = __builtin_bit_cast(v2u32, y);
    return (v4u32){x2[0], x2[1], y2[0], y2[1]};
}

// Store 32 rows x 64 dims held transposed in two accumulators (acc[ct]: lane
// (row ql, half hh) holds columns 32ct + acc_row(r, hh)), times `mul`.
template <int DT>
__device__ inline void store_rows(uint16_t* __restrict__ row_ptr, const v16f32 (&acc)[2],
                                  float mul, int hh) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            v2u32 w;
            w[0] = pack2<DT>(acc[ct][4 * g] * mul, acc[ct][4 * g + 1] * mul);
            w[1] = pack2<DT>(acc[ct][4 * g + 2] * mul, acc[ct][4 * g + 3] * mul);
            *(v2u32*)(row_ptr + 32 * ct + acc_row(4 * g, hh)) = w;
        }
}

}  // namespace attn
