// The gated linear recurrence for gfx950: per (batch, head) a D x D state S
// that each step scales column by column with the gate and grows by the
// outer product of k and v, read out through q (the recurrence the
// POPCORNBENCH transcript "Kimi-K2.6 l2 p24" analyses):
//   S[i][j] <- gate[t][j] * S[i][j] + k[t][i] * v[t][j],
//   y[t][j]  = sum_i q[t][i] * S[i][j],
// with q, k, v, gate and y in [B, T, H, D] float32, as on that page.
//
// gfx950 design (the page's kernels give each column to one CUDA thread that
// loops over the rows):
//  - One wave64 owns 8 columns of one (batch, head): lane = 8 * column + g,
//    and lane g of a column keeps the rows i = g, g + 8, ... (NI = ceil(D/8)
//    of them) of that column in registers. The state never leaves
//    registers; the only chain carried from step to step is one FMA per
//    state element.
//  - The readout sum over i is each lane's NI products, then a sum over the
//    column's 8 lanes by three DPP adds (quad_perm twice, row_half_mirror):
//    no LDS, no barrier, and waves never wait for each other.
//  - The inputs of a block of U steps are loaded into registers while the
//    previous block computes (q, k: the lane's NI rows; v, gate: its
//    column), so the loads' latency hides under the arithmetic.
//  - Rows past D carry k = 0 (their state stays 0); columns past D and
//    steps past T compute on in-bounds data and are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace attn {

// x plus the value of lane l ^ 1, then of l ^ 2 (within each quad), then of
// the mirror lane within each group of 8: after the three steps every lane
// of a group of 8 holds the group's sum.
__device__ inline float sum8(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                            0xf, 0xf, true));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>());   // quad_perm [1, 0, 3, 2]
    x += dpp(x, std::integral_constant<int, 0x4E>());   // quad_perm [2, 3, 0, 1]
    x += dpp(x, std::integral_constant<int, 0x141>());  // row_half_mirror
    return x;
}

// A raw buffer resource over `bytes` bytes from `base` (wave-uniform).
__device__ inline __amdgpu_buffer_rsrc_t slice_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
// One float at byte voff (per lane) + soff (wave-uniform) of a buffer.
__device__ inline float load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// One wave per (slice, 8-column block); grid = B * H * ceil(D / 8) waves.
// The caller guarantees T * H * D * 4 < 2^31 (byte offsets are 32-bit).
template <int NI, int U>
__global__ __launch_bounds__(64) void gated_recurrence32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ gate, float* __restrict__ y, int T, int H, int D, int jblocks) {
    const int lane = threadIdx.x;
    const int g = lane & 7;
    const int unit = blockIdx.x;
    const int bh = unit / jblocks;
    const int j = (unit - bh * jblocks) * 8 + (lane >> 3);
    const int b = bh / H, h = bh - b * H;
    const bool col_ok = j < D;
    // element (b, t, h, e) sits at ((b * T + t) * H + h) * D + e
    const int64_t step_stride = (int64_t)H * D;
    const int64_t base = ((int64_t)b * T * H + h) * D;

    float S[NI];
#pragma unroll
    for (int r = 0; r < NI; ++r) S[r] = 0.f;

    struct Block {
        float q[U][NI], k[U][NI], v[U], g[U];
    };
    // Every load stays in bounds: steps past T re-read step T - 1 (their
    // results are never stored), rows and columns past D re-read row or
    // column D - 1, and a row past D gets k = 0, so its state stays 0 and
    // adds nothing to the readout. The step's address is wave-uniform and
    // the lane's offset fixed, so each load is a scalar base plus one
    // 32-bit lane offset.
    // Loads go through buffer resources over the slice's extent (steps
    // 0 .. T-1 of head h of batch b), with the step's byte offset as a
    // scalar and the lane's byte offset as its one address register.
    const uint32_t extent = (uint32_t)(((int64_t)(T - 1) * step_stride + D) * 4);
    const __amdgpu_buffer_rsrc_t qr = slice_rsrc(q + base, extent);
    const __amdgpu_buffer_rsrc_t kr = slice_rsrc(k + base, extent);
    const __amdgpu_buffer_rsrc_t vr = slice_rsrc(v + base, extent);
    const __amdgpu_buffer_rsrc_t gr = slice_rsrc(gate + base, extent);
    int ioff[NI];
    bool row_ok[NI];
#pragma unroll
    for (int r = 0; r < NI; ++r) {
        const int i = g + 8 * r;
        ioff[r] = 4 * (i < D ? i : D - 1);
        row_ok[r] = i < D;
    }
    const int joff = 4 * (col_ok ? j : D - 1);
    const int step_bytes = (int)(step_stride * 4);
    auto load = [&](Block& blk, int t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int soff = min(t0 + u, T - 1) * step_bytes;
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                blk.q[u][r] = load_f32(qr, ioff[r], soff);
                const float kx = load_f32(kr, ioff[r], soff);
                blk.k[u][r] = row_ok[r] ? kx : 0.f;
            }
            blk.v[u] = load_f32(vr, joff, soff);
            blk.g[u] = load_f32(gr, joff, soff);
        }
    };
    auto compute = [&](const Block& blk, int t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                S[r] = fmaf(blk.g[u], S[r], blk.k[u][r] * blk.v[u]);
                acc = fmaf(blk.q[u][r], S[r], acc);
            }
            acc = sum8(acc);
            const int t = t0 + u;
            if (g == (u & 7) && col_ok && t < T) y[base + (int64_t)t * step_stride + j] = acc;
        }
    };

    // two register blocks in turn: block n + 1 loads while block n computes
    Block a, c;
    load(a, 0);
    for (int t0 = 0; t0 < T; t0 += 2 * U) {
        if (t0 + U < T) load(c, t0 + U);
        compute(a, t0);
        if (t0 + U >= T) break;
        if (t0 + 2 * U < T) load(a, t0 + 2 * U);
        compute(c, t0 + U);
    }
}

template <int NI>
static const void* rec_ptr() {
    return (const void*)gated_recurrence32<NI, (NI <= 4 ? 8 : 4)>;
}

const void* recurrence_kernel_ptr(int index) {
    switch (index) {
        case 0: return rec_ptr<1>();
        case 1: return rec_ptr<2>();
        case 2: return rec_ptr<3>();
        case 3: return rec_ptr<4>();
        case 4: return rec_ptr<5>();
        case 5: return rec_ptr<6>();
        case 6: return rec_ptr<7>();
        case 7: return rec_ptr<8>();
        default: return nullptr;
    }
}

hipError_t launch_recurrence(const float* q, const float* k, const float* v, const float* gate,
                             float* y, int B, int T, int H, int D, hipStream_t stream) {
    const int ni = (D + 7) / 8;
    const void* fn = recurrence_kernel_ptr(ni - 1);
    if (fn == nullptr) return hipErrorInvalidValue;
    int jblocks = ni;  // 8 columns per wave
    const dim3 grid((unsigned)((int64_t)B * H * jblocks));
    const dim3 block(64);
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&gate, (void*)&y,
                    (void*)&T, (void*)&H, (void*)&D, (void*)&jblocks};
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace attn
