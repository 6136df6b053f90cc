// The materialising contrast path, fp32: the T x T score table is written to
// device memory, swept by a safe softmax into a second T x T table, and then
// weighed against V. It follows the three-kernel path of the page
// "attention.cu" (a tiled Q K^T, a max pass and an exp-and-sum pass per row,
// and a tiled P V that divides by the row sums): five passes over 4*T*T bytes
// per head. Its only job is the memory contrast with the fused path, so it is
// a reasonable tiled implementation (LDS tiles, 4x4 outputs per thread), not
// a tuned one, and it runs on the vector ALUs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

namespace {

constexpr int kD = 64;       // head dimension
constexpr int kTile = 64;    // output tile edge (rows and columns)
constexpr int kPad = 68;     // LDS row stride in floats (16-byte aligned)
constexpr int kRowThreads = 256;

// S[bh, i, j] = scale * sum_e Q[bh, i, e] * K[bh, j, e] for a 64 x 64 tile.
// grid (ceil(T/64) column tiles, ceil(T/64) row tiles, BH); 256 threads.
__global__ __launch_bounds__(256) void naive_scores(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    float* __restrict__ s, int T,
                                                    float scale) {
    __shared__ __attribute__((aligned(16))) float qt[kD][kPad];  // [e][i]
    __shared__ __attribute__((aligned(16))) float kt[kD][kPad];  // [e][j]
    const int tid = threadIdx.x;
    const int j0 = blockIdx.x * kTile, i0 = blockIdx.y * kTile;
    const int64_t bh = blockIdx.z;
    const float* qh = q + bh * T * kD;
    const float* kh = k + bh * T * kD;
    for (int n = 0; n < 4; ++n) {
        const int idx = tid + 256 * n;  // 1024 float4 chunks per tile
        const int row = idx >> 4, e4 = (idx & 15) * 4;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (i0 + row < T) a = *(const float4*)(qh + (int64_t)(i0 + row) * kD + e4);
        if (j0 + row < T) b = *(const float4*)(kh + (int64_t)(j0 + row) * kD + e4);
        qt[e4 + 0][row] = a.x; qt[e4 + 1][row] = a.y;
        qt[e4 + 2][row] = a.z; qt[e4 + 3][row] = a.w;
        kt[e4 + 0][row] = b.x; kt[e4 + 1][row] = b.y;
        kt[e4 + 2][row] = b.z; kt[e4 + 3][row] = b.w;
    }
    __syncthreads();
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int e = 0; e < kD; ++e) {
        const float4 a = *(const float4*)&qt[e][4 * ty];
        const float4 b = *(const float4*)&kt[e][4 * tx];
        const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        for (int x = 0; x < 4; ++x)
            for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
    }
    float* sh = s + bh * (int64_t)T * T;
    for (int x = 0; x < 4; ++x) {
        const int i = i0 + 4 * ty + x;
        if (i >= T) continue;
        for (int y = 0; y < 4; ++y) {
            const int j = j0 + 4 * tx + y;
            if (j < T) sh[(int64_t)i * T + j] = acc[x][y] * scale;
        }
    }
}

__device__ inline float block_reduce(float x, bool is_max, float* scratch) {
    for (int off = 32; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) scratch[wave] = x;
    __syncthreads();
    float r = scratch[0];
    for (int w = 1; w < kRowThreads / 64; ++w)
        r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
    __syncthreads();
    return r;
}

// One row per workgroup: a pass for the maximum over the visible keys, then a
// pass that writes exp(s - max) (0 for masked keys) to P and totals it.
// grid (T, BH); 256 threads.
__global__ __launch_bounds__(kRowThreads) void naive_softmax(
    const float* __restrict__ s, float* __restrict__ p,
    float* __restrict__ rowsum, float* __restrict__ lse, int T, int causal) {
    __shared__ float scratch[kRowThreads / 64];
    const int i = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int64_t row = bh * T + i;
    const float* line = s + row * T;
    float* out = p + row * T;
    const int visible = causal ? i + 1 : T;
    float best = -INFINITY;
    for (int j = threadIdx.x; j < visible; j += kRowThreads)
        best = fmaxf(best, line[j]);
    best = block_reduce(best, true, scratch);
    float total = 0.f;
    for (int j = threadIdx.x; j < T; j += kRowThreads) {
        const float e = j < visible ? expf(line[j] - best) : 0.f;
        out[j] = e;
        total += e;
    }
    total = block_reduce(total, false, scratch);
    if (threadIdx.x == 0) {
        rowsum[row] = total;
        if (lse != nullptr) lse[row] = best + logf(total);
    }
}

// O[bh, i, :] = (sum_j P[bh, i, j] V[bh, j, :]) / rowsum[bh, i] for 64 rows.
// grid (ceil(T/64), BH); 256 threads.
__global__ __launch_bounds__(256) void naive_weighted_v(
    const float* __restrict__ p, const float* __restrict__ v,
    const float* __restrict__ rowsum, float* __restrict__ o, int T) {
    __shared__ __attribute__((aligned(16))) float pt[kTile][kPad];  // [j][i]
    __shared__ __attribute__((aligned(16))) float vs[kTile][kPad];  // [j][d]
    const int tid = threadIdx.x;
    const int i0 = blockIdx.x * kTile;
    const int64_t bh = blockIdx.y;
    const float* ph = p + bh * (int64_t)T * T;
    const float* vh = v + bh * (int64_t)T * kD;
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int j0 = 0; j0 < T; j0 += kTile) {
        for (int n = 0; n < 16; ++n) {  // 4096 P values, scalar (rows of T)
            const int idx = tid + 256 * n;
            const int r = idx >> 6, cc = idx & 63;
            float x = 0.f;
            if (i0 + r < T && j0 + cc < T) x = ph[(int64_t)(i0 + r) * T + j0 + cc];
            pt[cc][r] = x;
        }
        for (int n = 0; n < 4; ++n) {
            const int idx = tid + 256 * n;
            const int r = idx >> 4, d4 = (idx & 15) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j0 + r < T) x = *(const float4*)(vh + (int64_t)(j0 + r) * kD + d4);
            *(float4*)&vs[r][d4] = x;
        }
        __syncthreads();
        for (int j = 0; j < kTile; ++j) {
            const float4 a = *(const float4*)&pt[j][4 * ty];
            const float4 b = *(const float4*)&vs[j][4 * tx];
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
            for (int x = 0; x < 4; ++x)
                for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
        }
        __syncthreads();
    }
    for (int x = 0; x < 4; ++x) {
        const int i = i0 + 4 * ty + x;
        if (i >= T) continue;
        const float inv = 1.0f / rowsum[bh * T + i];
        float4 w = make_float4(acc[x][0] * inv, acc[x][1] * inv, acc[x][2] * inv,
                               acc[x][3] * inv);
        *(float4*)(o + (bh * T + i) * kD + 4 * tx) = w;
    }
}

}  // namespace

hipError_t launch_naive(const float* q, const float* k, const float* v,
                        float* o, float* lse, float* s, float* p,
                        float* rowsum, int BH, int T, int causal, float scale,
                        hipStream_t stream) {
    const unsigned nt = (unsigned)((T + kTile - 1) / kTile);
    hipLaunchKernelGGL(naive_scores, dim3(nt, nt, BH), dim3(256), 0, stream, q,
                       k, s, T, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(naive_softmax, dim3((unsigned)T, BH), dim3(kRowThreads),
                       0, stream, s, p, rowsum, lse, T, causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(naive_weighted_v, dim3(nt, BH), dim3(256), 0, stream, p,
                       v, rowsum, o, T);
    return hipGetLastError();
}

const void* naive_kernel_ptr(int index) {
    switch (index) {
        case 0: return (const void*)naive_scores;
        case 1: return (const void*)naive_softmax;
        case 2: return (const void*)naive_weighted_v;
        default: return nullptr;
    }
}

}  // namespace attn
