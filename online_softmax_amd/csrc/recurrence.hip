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
//  - One workgroup per (batch, head); one wave64 owns 8 columns: lane =
//    8 * column + g, and lane g of a column keeps the rows i = g, g + 8, ...
//    (NI = ceil(D/8) of them) of that column in registers. The state never
//    leaves registers; the only chain carried from step to step is one FMA
//    per state element.
//  - The readout sum over i is each lane's NI products, then a sum over the
//    column's 8 lanes by three DPP adds (quad_perm twice, row_half_mirror).
//  - With many (batch, head) slices, inputs go through LDS in blocks of
//    steps, loaded once per workgroup with coalesced loads while the
//    previous block computes; with few, each wave prefetches its own inputs
//    into registers (no barrier, nothing between a load and its use but the
//    arithmetic). Details at each kernel.
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

// Few (batch, head) slices (too few workgroups to fill the GPU): latency
// decides, so each wave loads its own inputs straight into registers, a
// block of U steps ahead, with no LDS and no barrier. One wave per (slice,
// 8-column block); grid = B * H * ceil(D / 8) waves. The caller guarantees
// T * H * D * 4 < 2^31 (byte offsets are 32-bit).
template <int NI, int U>
__global__ __launch_bounds__(64) void gated_recurrence_wave32(
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

// Many slices (throughput): one workgroup per (batch, head), one wave per 8
// columns (NI = ceil(D/8) waves of 64 lanes; D <= 64). The steps go in blocks of kRecSteps: a block
// of q, k, v and the gate (every row of the slice's steps, read once,
// coalesced, by the whole workgroup) is staged in LDS while the previous
// block computes, so each wave reads its inputs from LDS instead of
// fetching q and k again per wave. In LDS, q and k of a step are stored
// with element i at 8 (i mod 8) + i / 8, so lane g's rows g, g + 8, ... are
// 8 consecutive floats (two 16-byte reads); v and the gate keep their
// column order. Rows and columns past D hold 0 (written once), so their
// state stays 0; steps past T hold 0 and are never stored.
constexpr int kRecSteps = 16;
// from this many (batch, head) slices on, the workgroup kernel runs (every
// CU gets at least half a workgroup); below, the per-wave kernel
constexpr int kRecWorkgroupSlices = 128;
constexpr int kRecSlots = 64;  // padded row of one step

template <int NI>
__global__ __launch_bounds__(64 * NI) void gated_recurrence32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ gate, float* __restrict__ y, int T, int H, int D) {
    constexpr int kThreadsR = 64 * NI;
    constexpr int kBlockElems = 4 * kRecSteps * kRecSlots;
    // elements a block loads: 4 tensors x kRecSteps steps x D <= 8 NI
    constexpr int kPerThread = (4 * kRecSteps * 8 * NI + kThreadsR - 1) / kThreadsR;
    __shared__ __attribute__((aligned(16))) float lds[2][4][kRecSteps][kRecSlots];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = lane & 7;
    const int j = (tid >> 6) * 8 + (lane >> 3);  // this lane's column
    const bool col_ok = j < D;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    // element (b, t, h, e) sits at ((b * T + t) * H + h) * D + e
    const int64_t step_stride = (int64_t)H * D;
    const int64_t base = ((int64_t)b * T * H + h) * D;
    const float* src[4] = {q + base, k + base, v + base, gate + base};

    // zero both stages once: the slots past D are never written again
    for (int e = tid; e < 2 * kBlockElems; e += kThreadsR) (&lds[0][0][0][0])[e] = 0.f;

    // thread tid carries elements tid + n * kThreadsR of a block: tensor x,
    // step u, element i (< D only); loaded into registers, then written to
    // their LDS slots. The split of an element index into (x, u, i) is the
    // same for every block, so it is made once: the element's address in
    // block 0, its step u (-1: the thread has no element n) and its slot.
    const int per_block = 4 * kRecSteps * D;
    const float* lp[kPerThread];
    int lu[kPerThread], lpos[kPerThread];
#pragma unroll
    for (int n = 0; n < kPerThread; ++n) {
        const int e = tid + n * kThreadsR;
        lp[n] = src[0];
        lu[n] = -1;
        lpos[n] = 0;
        if (e < per_block) {
            const int x = e / (kRecSteps * D);
            const int rem = e - x * (kRecSteps * D);
            const int u = rem / D;
            const int i = rem - u * D;
            lp[n] = src[x] + (int64_t)u * step_stride + i;
            lu[n] = u;
            lpos[n] = (x * kRecSteps + u) * kRecSlots + (x < 2 ? 8 * (i & 7) + (i >> 3) : i);
        }
    }
    const int64_t block_stride = (int64_t)kRecSteps * step_stride;
    float buf[kPerThread];
    auto load = [&](int blk) {
#pragma unroll
        for (int n = 0; n < kPerThread; ++n) {
            const int t = blk * kRecSteps + lu[n];
            buf[n] = (lu[n] >= 0 && t < T) ? lp[n][blk * block_stride] : 0.f;
        }
    };
    auto stage = [&](int slot) {
        float* st = &lds[slot][0][0][0];
#pragma unroll
        for (int n = 0; n < kPerThread; ++n)
            if (lu[n] >= 0) st[lpos[n]] = buf[n];
    };

    float S[NI];
#pragma unroll
    for (int r = 0; r < NI; ++r) S[r] = 0.f;
    // One step's inputs as the lane reads them: its 8 rows of q and of k,
    // v and the gate of its column. The next step's are read before this
    // step computes, so LDS latency hides behind the arithmetic.
    struct StepIn {
        float4 q0, q1, k0, k1;
        float v, g;
    };
    auto read = [&](int slot, int u, StepIn& x) {
        const float4* qrow = (const float4*)&lds[slot][0][u][8 * g];
        const float4* krow = (const float4*)&lds[slot][1][u][8 * g];
        x.q0 = qrow[0];
        x.q1 = qrow[1];
        x.k0 = krow[0];
        x.k1 = krow[1];
        x.v = lds[slot][2][u][j];
        x.g = lds[slot][3][u][j];
    };
    auto compute = [&](int slot, int t0) {
        StepIn cur, nxt;
        read(slot, 0, cur);
#pragma unroll
        for (int u = 0; u < kRecSteps; ++u) {
            if (u + 1 < kRecSteps) read(slot, u + 1, nxt);
            const float qv[8] = {cur.q0.x, cur.q0.y, cur.q0.z, cur.q0.w,
                                 cur.q1.x, cur.q1.y, cur.q1.z, cur.q1.w};
            const float kv[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w,
                                 cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                S[r] = fmaf(cur.g, S[r], kv[r] * cur.v);
                acc = fmaf(qv[r], S[r], acc);
            }
            acc = sum8(acc);
            const int t = t0 + u;
            if (g == (u & 7) && col_ok && t < T) y[base + (int64_t)t * step_stride + j] = acc;
            if (u + 1 < kRecSteps) cur = nxt;
        }
    };

    const int nblk = (T + kRecSteps - 1) / kRecSteps;
    __syncthreads();  // the zeroing is done before any stage writes
    load(0);
    stage(0);
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const bool more = blk + 1 < nblk;
        if (more) load(blk + 1);  // in flight while this block computes
        compute(blk & 1, blk * kRecSteps);
        if (more) stage((blk + 1) & 1);  // that stage was last read a block ago
        __syncthreads();
    }
}

template <int NI>
static const void* rec_ptr(bool per_wave) {
    return per_wave ? (const void*)gated_recurrence_wave32<NI, (NI <= 4 ? 8 : 4)>
                    : (const void*)gated_recurrence32<NI>;
}

// Table: entries 0 .. 7 the workgroup kernel for NI = 1 .. 8, entries
// 8 .. 15 the per-wave kernel.
const void* recurrence_kernel_ptr(int index) {
    if (index < 0 || index >= 16) return nullptr;
    const bool w = index >= 8;
    switch (index & 7) {
        case 0: return rec_ptr<1>(w);
        case 1: return rec_ptr<2>(w);
        case 2: return rec_ptr<3>(w);
        case 3: return rec_ptr<4>(w);
        case 4: return rec_ptr<5>(w);
        case 5: return rec_ptr<6>(w);
        case 6: return rec_ptr<7>(w);
        case 7: return rec_ptr<8>(w);
        default: return nullptr;
    }
}

hipError_t launch_recurrence(const float* q, const float* k, const float* v, const float* gate,
                             float* y, int B, int T, int H, int D, hipStream_t stream) {
    const int ni = (D + 7) / 8;  // 8 columns per wave
    if ((int64_t)B * H < kRecWorkgroupSlices) {
        const void* fn = recurrence_kernel_ptr(8 + ni - 1);
        if (fn == nullptr) return hipErrorInvalidValue;
        int jblocks = ni;
        const dim3 grid((unsigned)((int64_t)B * H * jblocks));
        void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&gate, (void*)&y,
                        (void*)&T, (void*)&H, (void*)&D, (void*)&jblocks};
        return hipLaunchKernel(fn, grid, dim3(64), args, 0, stream);
    }
    const void* fn = recurrence_kernel_ptr(ni - 1);
    if (fn == nullptr) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((int64_t)B * H));
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&gate, (void*)&y,
                    (void*)&T, (void*)&H, (void*)&D};
    return hipLaunchKernel(fn, grid, dim3(64 * ni), args, 0, stream);
}

}  // namespace attn
