// Fused attention forward for gfx950: the online softmax over key tiles,
// computed on the matrix cores, with the T x T score table never stored.
//
// Per query row the kernel keeps a running maximum m, a running denominator l
// and a running output, and when a key tile brings a larger maximum it
// multiplies l and the output by exp(m_old - m_new) before adding the tile's
// own terms ("Flash attention in PyTorch, then in Triton", section "Flash
// attention"; the same update is the online-state loop of the fused kernel of
// the page "attention.cu"). Exponentials are taken as exp2 with log2(e) and
// the scale folded into one multiplier (section "A kernel in Triton"), the
// causal loop stops at the query tile's last row, which skips about half the
// key tiles (section "The online softmax, in PyTorch"), and each row's
// log-sum-exp is written alongside the output (section "Backwards, and
// training with it").
//
// gfx950 design (not the pages' - their kernels were written for a T4 and an
// RTX 4090):
//  - 4 wave64s per workgroup, 32 query rows per wave, 128 per workgroup.
//  - Q fragments live in VGPRs for the whole kernel.
//  - K and V tiles go global -> VGPRs -> LDS with 128-bit loads, double
//    buffered in padded LDS (one barrier per tile); the next tile's global
//    loads are in flight while the current tile computes. V is transposed on
//    its way into LDS so the PV product reads 16-byte fragments.
//  - S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}
//    (fp32 inputs: v_mfma_f32_32x32x2_f32), fp32 accumulation.
//  - Row max / row sum: in-lane, then one v_permlane32_swap between halves.
//  - Masks only on the diagonal and ragged tiles; tiles a whole wave cannot
//    see are skipped by that wave (it still joins every barrier).
// Index arithmetic lives in fused_layout.h (host-checkable).
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fused_layout.h"
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

// ---------------------------------------------------------------------------
// 16-bit inputs (bf16 or f16), fp32 accumulation.
// c = |scale| * log2(e); qsign = 0x80008000 negates Q for a negative scale.
// ---------------------------------------------------------------------------
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fused_fwd16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    constexpr int BN = kBlockN16;
    __shared__ __attribute__((aligned(16))) uint16_t sk[2][kKTile16];
    __shared__ __attribute__((aligned(16))) uint16_t sv[2][kVTile16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const uint16_t* qh = q + base;
    const uint16_t* kh = k + base;
    const uint16_t* vh = v + base;
    const int wq0 = qt * kBlockM + 32 * wave;  // first query row of this wave
    const int my_q = wq0 + ql;                 // this lane's query row
    const int n_tiles = key_tiles(qt, T, BN, CAUSAL);

    v4u32 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T)
            x = *(const v4u32*)(qh + (int64_t)my_q * kHeadDim + q_col16(hh, ks));
        qf[ks] = x ^ qsign;
    }

    v4u32 kr[2], vr[2];
    auto gload = [&](int kt) {
        const int k0 = kt * BN;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage16(tid, i, &row, &col);
            v4u32 x = {0u, 0u, 0u, 0u};
            if (k0 + row < T)
                x = *(const v4u32*)(kh + (int64_t)(k0 + row) * kHeadDim + col);
            kr[i] = x;
        }
        int key0, dim0;
        v_stage16(tid, &key0, &dim0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            v4u32 x = {0u, 0u, 0u, 0u};
            if (k0 + key0 + e < T)
                x = *(const v4u32*)(vh + (int64_t)(k0 + key0 + e) * kHeadDim +
                                    dim0);
            vr[e] = x;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage16(tid, i, &row, &col);
            *(v4u32*)&sk[buf][k_lds16(row, col)] = kr[i];
        }
        int key0, dim0;
        v_stage16(tid, &key0, &dim0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = vr[0][j], b = vr[1][j];
            // dims dim0 + 2j and dim0 + 2j + 1, each as (key0, key0 + 1)
            *(uint32_t*)&sv[buf][v_lds16(dim0 + 2 * j, key0)] =
                (a & 0xffffu) | (b << 16);
            *(uint32_t*)&sv[buf][v_lds16(dim0 + 2 * j + 1, key0)] =
                (a >> 16) | (b & 0xffff0000u);
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    v16f32 oacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    float m = -FLT_MAX;  // running max of raw scores (finite start: no inf-inf)
    float l = 0.f;       // running denominator, this lane-half's keys only

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) gload(kt + 1);
        const int k0 = kt * BN;
        // a wave skips tiles none of its rows can see (still joins barriers)
        if (!CAUSAL || k0 <= wq0 + 31) {
            v16f32 s[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    s[nt] = mfma16<DT>(
                        *(const v4u32*)&sk[buf][kfrag16(ql, hh, nt, ks)],
                        qf[ks], s[nt]);
            }
            const bool edge =
                (CAUSAL && k0 + BN - 1 > wq0) || (k0 + BN > T);
            if (edge) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * nt + acc_row(r, hh);
                        if (key >= T || (CAUSAL && key > my_q))
                            s[nt][r] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
            mx = halves_max(mx);
            const float m_new = fmaxf(m, mx);
            const float mc = m_new * c;
            const float corr = fast_exp2(m * c - mc);
            m = m_new;
            float rs = 0.f;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(s[nt][r], c, -mc));
                    if (edge && s[nt][r] == -INFINITY) p = 0.f;
                    s[nt][r] = p;
                    rs += p;
                }
            l = l * corr + rs;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
            v4u32 pf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int nt = ks >> 1, r0 = (ks & 1) * 8;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pf[ks][i] =
                        pack2<DT>(s[nt][r0 + 2 * i], s[nt][r0 + 2 * i + 1]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    oacc[mt] = mfma16<DT>(
                        *(const v4u32*)&sv[buf][vfrag16(ql, hh, mt, ks)],
                        pf[ks], oacc[mt]);
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    const float lt = halves_sum(l);
    const float inv = 1.0f / lt;
    if (my_q < T) {
        uint16_t* orow = o + base + (int64_t)my_q * kHeadDim;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v2u32 w;
                w[0] = pack2<DT>(oacc[mt][4 * g] * inv, oacc[mt][4 * g + 1] * inv);
                w[1] = pack2<DT>(oacc[mt][4 * g + 2] * inv,
                                 oacc[mt][4 * g + 3] * inv);
                *(v2u32*)(orow + 32 * mt + acc_row(4 * g, hh)) = w;
            }
        if (lse != nullptr && hh == 0)
            lse[(int64_t)bh * T + my_q] = (m * c + log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same schedule on v_mfma_f32_32x32x2_f32, 32-key tiles.
// qsign = 0x80000000 negates Q for a negative scale.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fused_fwd32(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    constexpr int BN = kBlockN32;
    __shared__ __attribute__((aligned(16))) float sk[2][kKTile32];
    __shared__ __attribute__((aligned(16))) float sv[2][kVTile32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const float* qh = q + base;
    const float* kh = k + base;
    const float* vh = v + base;
    const int wq0 = qt * kBlockM + 32 * wave;
    const int my_q = wq0 + ql;
    const int n_tiles = key_tiles(qt, T, BN, CAUSAL);

    v4f32 qf[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T)
            x = *(const v4u32*)(qh + (int64_t)my_q * kHeadDim + q_col32(hh, g));
        qf[g] = __builtin_bit_cast(v4f32, x ^ qsign);
    }

    v4f32 kr[2], vr[2];
    auto gload = [&](int kt) {
        const int k0 = kt * BN;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage32(tid, i, &row, &col);
            v4f32 x = {0.f, 0.f, 0.f, 0.f};
            if (k0 + row < T)
                x = *(const v4f32*)(kh + (int64_t)(k0 + row) * kHeadDim + col);
            kr[i] = x;
        }
        int key0, dim0;
        v_stage32(tid, &key0, &dim0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            v4f32 x = {0.f, 0.f, 0.f, 0.f};
            if (k0 + key0 + e < T)
                x = *(const v4f32*)(vh + (int64_t)(k0 + key0 + e) * kHeadDim +
                                    dim0);
            vr[e] = x;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage32(tid, i, &row, &col);
            *(v4f32*)&sk[buf][k_lds32(row, col)] = kr[i];
        }
        int key0, dim0;
        v_stage32(tid, &key0, &dim0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float2 w;
            w.x = vr[0][j];
            w.y = vr[1][j];
            *(float2*)&sv[buf][v_lds32(dim0 + j, key0)] = w;
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    v16f32 oacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    float m = -FLT_MAX;
    float l = 0.f;

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) gload(kt + 1);
        const int k0 = kt * BN;
        if (!CAUSAL || k0 <= wq0 + 31) {
            v16f32 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const v4f32 kf = *(const v4f32*)&sk[buf][kfrag32(ql, hh, g)];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i], qf[g][i], s,
                                                              0, 0, 0);
            }
            const bool edge =
                (CAUSAL && k0 + BN - 1 > wq0) || (k0 + BN > T);
            if (edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + acc_row(r, hh);
                    if (key >= T || (CAUSAL && key > my_q)) s[r] = -INFINITY;
                }
            }
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = halves_max(mx);
            const float m_new = fmaxf(m, mx);
            const float mc = m_new * c;
            const float corr = fast_exp2(m * c - mc);
            m = m_new;
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[r], c, -mc));
                if (edge && s[r] == -INFINITY) p = 0.f;
                s[r] = p;
                rs += p;
            }
            l = l * corr + rs;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
            // O^T += V^T P^T: step 4g + i pairs key 8g + 4h + i of each half
            // with accumulator register 4g + i of the score tile.
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v4f32 vf =
                        *(const v4f32*)&sv[buf][vfrag32(ql, hh, mt, g)];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            vf[i], s[4 * g + i], oacc[mt], 0, 0, 0);
                }
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    const float lt = halves_sum(l);
    const float inv = 1.0f / lt;
    if (my_q < T) {
        float* orow = o + base + (int64_t)my_q * kHeadDim;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v4f32 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = oacc[mt][4 * g + i] * inv;
                *(v4f32*)(orow + 32 * mt + acc_row(4 * g, hh)) = w;
            }
        if (lse != nullptr && hh == 0)
            lse[(int64_t)bh * T + my_q] = (m * c + log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Launchers and the kernel table.
// ---------------------------------------------------------------------------
hipError_t launch_fused(const void* q, const void* k, const void* v, void* o,
                        float* lse, int BH, int T, int causal, float c,
                        bool negate_q, int dt, hipStream_t stream) {
    const int nq = (T + kBlockM - 1) / kBlockM;
    const dim3 grid((unsigned)(nq * BH));
    const dim3 block(kThreads);
    if (dt == ATTN_DT_F32) {
        const uint32_t sign = negate_q ? 0x80000000u : 0u;
        auto fn = causal ? fused_fwd32<true> : fused_fwd32<false>;
        hipLaunchKernelGGL(fn, grid, block, 0, stream, (const float*)q,
                           (const float*)k, (const float*)v, (float*)o, lse, T,
                           nq, c, sign);
    } else {
        const uint32_t sign = negate_q ? 0x80008000u : 0u;
        if (dt == ATTN_DT_BF16) {
            auto fn = causal ? fused_fwd16<ATTN_DT_BF16, true>
                             : fused_fwd16<ATTN_DT_BF16, false>;
            hipLaunchKernelGGL(fn, grid, block, 0, stream, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v,
                               (uint16_t*)o, lse, T, nq, c, sign);
        } else {
            auto fn = causal ? fused_fwd16<ATTN_DT_F16, true>
                             : fused_fwd16<ATTN_DT_F16, false>;
            hipLaunchKernelGGL(fn, grid, block, 0, stream, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v,
                               (uint16_t*)o, lse, T, nq, c, sign);
        }
    }
    return hipGetLastError();
}

const void* fused_kernel_ptr(int index) {
    switch (index) {
        case 0: return (const void*)fused_fwd16<ATTN_DT_BF16, true>;
        case 1: return (const void*)fused_fwd16<ATTN_DT_BF16, false>;
        case 2: return (const void*)fused_fwd16<ATTN_DT_F16, true>;
        case 3: return (const void*)fused_fwd16<ATTN_DT_F16, false>;
        case 4: return (const void*)fused_fwd32<true>;
        case 5: return (const void*)fused_fwd32<false>;
        default: return nullptr;
    }
}

}  // namespace attn
