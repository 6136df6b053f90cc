// Fused attention forward for head dimensions other than 64 (32 and 128),
// 16-bit inputs: the same online softmax as the D = 64 kernel (running
// maximum, running denominator and rescaled output per query row, exp2 with
// the scale folded in, causal tiles beyond the query tile skipped, the
// log-sum-exp written beside O; "Flash attention in PyTorch, then in Triton",
// sections "Flash attention" and "A kernel in Triton"), with the head
// dimension a template parameter, as the pages' own kernels take it as a
// compile-time constant.
//
// gfx950 design:
//  - 4 wave64s per workgroup, 32 query rows per wave (128 per workgroup);
//    Q fragments (D / 16 of them) stay in VGPRs.
//  - K and V tiles of 64 keys x D arrive by direct buffer loads into LDS
//    rings: one barrier per tile, after which the next tile's loads are
//    issued and run under this tile's compute. Two workgroups per CU, so the
//    other workgroup's waves fill the matrix cores while a wave does its
//    softmax.
//  - D = 32 runs each tile's S, weights and P.V in order (two stages each
//    for K and V, 16 KiB). D = 128 skews the loop by one tile: the weights of
//    tile t are made while tile t-1's P.V products run, so one wave's vector
//    and matrix work overlap too (V in three stages: 80 KiB).
//  - S^T = K Q^T (D / 16 reduction steps) and O^T += V^T P^T (D / 32 output
//    tiles, V^T read with ds_read_b64_tr_b16), v_mfma_f32_32x32x16_{bf16,f16}.
//  - The per-D row swizzles and fragment addresses are HeadDim<D> in
//    fused_layout.h, checked on the host for coverage, decode and bank
//    conflicts.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fused_layout.h"
#include "gfx950.h"
#include "kernels.h"
#include "online_step.h"

namespace attn {

// S^T = K Q^T for one 64-key tile: kb the LDS tile, ko[ks] the lane's K
// fragment address at step ks (the second 32-key half adds 32 rows).
template <int DT, int D>
__device__ inline void qk_hd(const char* __restrict__ kb, const uint32_t (&ko)[D / 16],
                             const v4u32 (&qf)[D / 16], v16f32 (&s)[2]) {
    using G = HeadDim<D>;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::kSteps; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const v4u32 kf = *(const v4u32*)(kb + ko[ks] + 32 * G::kRowBytes * nt);
            s[nt] = mfma16<DT>(kf, qf[ks], s[nt]);
        }
}

// O^T += V^T P^T for one 64-key tile: vo[mt] the lane's transposed-read
// address of output tile mt (step ks adds 16 rows, the second half 8).
template <int DT, int D>
__device__ inline void pv_hd(const char* __restrict__ vb, const uint32_t (&vo)[D / 32],
                             const v4u32 (&pf)[4], v16f32 (&oacc)[D / 32]) {
    using G = HeadDim<D>;
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
#pragma unroll
    for (int mt = 0; mt < G::kOTiles; ++mt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const char* p = vb + vo[mt] + 16 * G::kRowBytes * ks;
            const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
            const v4i16 b =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * G::kRowBytes));
            const v2u32 a2 = __builtin_bit_cast(v2u32, a), b2 = __builtin_bit_cast(v2u32, b);
            const v4u32 vf = {a2[0], a2[1], b2[0], b2[1]};
            oacc[mt] = mfma16<DT>(vf, pf[ks], oacc[mt]);
        }
}

// Which head dimensions run the skewed loop (below): at D = 128 the 16
// products of a tile's P.V take about as long as its weights, so the two
// overlap; the third V stage fits two workgroups per CU (80 KiB each).
template <int D>
constexpr bool hd_skewed() { return D == 128; }

// Schedule of the skewed loop's unmasked step: the previous tile's P.V
// matrix instructions spread between the weights' vector instructions.
template <int NO>
__device__ inline void hd_sched_skewed() {
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
#pragma unroll
    for (int i = 0; i < 4 * NO; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 96 / (4 * NO), 0);    // VALU
    }
}

// Waves per SIMD the kernel is compiled for: D = 32 fits five (96 VGPRs,
// no spills; the causal kernel compiled for two took 97, four per SIMD, and
// ran 4-5% slower at 4 x 12 x 8192; six spill), D = 128 two.
template <int D>
constexpr int hd_waves_per_simd() { return D == 32 ? 5 : 2; }

// One workgroup: query tile qt (128 rows) of slice bh. c = |scale| log2(e);
// qsign negates Q for a negative scale.
template <int DT, bool CAUSAL, int D>
__global__ __launch_bounds__(kThreads, hd_waves_per_simd<D>()) void fused_hd16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    using G = HeadDim<D>;
    constexpr int BN = 64;
    constexpr int NK = G::kSteps, NO = G::kOTiles, NI = G::kInstrPerWave;
    constexpr bool SKEW = hd_skewed<D>();
    constexpr int kVStages = SKEW ? 3 : 2;
    __shared__ __attribute__((aligned(1024))) char kbuf[2][G::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char vbuf[kVStages][G::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * D;
    const uint16_t* qh = q + base;
    const int wq0 = qt * kBlockM + 32 * wave;
    const int my_q = wq0 + ql;
    const int n_tiles = key_tiles(qt, T, BN, CAUSAL);
    const int n_main = main_tiles(qt, T, BN, CAUSAL);

    // Direct loads: instruction wave * NI + i of a tile, lane's fixed offset
    // within the tile; the tile's offset is scalar. The ragged last tile
    // clamps rows past T to row T - 1 (weights of those keys are masked to
    // 0); the buffer's size (the slice) bounds every access in any case.
    const uint32_t slice_bytes = (uint32_t)T * G::kRowBytes;
    const v4u32_rsrc krs = buffer_rsrc(k + base, slice_bytes);
    const v4u32_rsrc vrs = buffer_rsrc(v + base, slice_bytes);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t kvoff[NI], vvoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        kvoff[i] = (uint32_t)G::global_byte(wave * NI + i, lane, false);
        vvoff[i] = (uint32_t)G::global_byte(wave * NI + i, lane, true);
    }
    auto load_tile = [&](v4u32_rsrc rs, const char* buf, const uint32_t(&voff)[NI],
                         int tile) {
        const uint32_t off = (uint32_t)(uintptr_t)(lds_void*)buf;
        const int k0 = __builtin_amdgcn_readfirstlane(tile) * BN;
        if (k0 + BN <= T) {
            const uint32_t soff = (uint32_t)k0 * G::kRowBytes;
#pragma unroll
            for (int i = 0; i < NI; ++i)
                dma16(rs, voff[i], soff, off + 1024 * (wave_u * NI + i));
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int r = min(k0 + (int)(voff[i] / G::kRowBytes), T - 1);
                dma16(rs, (uint32_t)r * G::kRowBytes + voff[i] % G::kRowBytes, 0u,
                      off + 1024 * (wave_u * NI + i));
            }
        }
    };
    // K tile t goes to stage t % 2, V tile t to stage t % kVStages
    auto issue = [&](int t) {
        load_tile(krs, kbuf[t & 1], kvoff, t);
        load_tile(vrs, vbuf[t % kVStages], vvoff, t);
    };
    if (n_tiles > 0) issue(0);

    v4u32 qf[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T) x = *(const v4u32*)(qh + (int64_t)my_q * D + G::q_col(hh, ks));
        qf[ks] = x ^ qsign;
    }
    uint32_t ko[NK], vo[NO];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) ko[ks] = (uint32_t)G::kfrag(ql, hh, 0, ks);
#pragma unroll
    for (int mt = 0; mt < NO; ++mt) vo[mt] = (uint32_t)G::vtr(lane, mt, 0, 0);

    v16f32 oacc[NO];
#pragma unroll
    for (int mt = 0; mt < NO; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    RowState st = {-FLT_MAX, -FLT_MAX * c, 0.f};

    // Plain order: iteration t waits for tile t, then S, weights and P.V of
    // tile t. Skewed order: iteration t waits only for K(t) (V(t), issued
    // after it, may still be in flight; loads complete in order, so V(t-1)
    // has landed), computes S(t), and makes tile t's weights while tile
    // t-1's P.V products run on the matrix cores; the last tile's product
    // follows the loop. K(t+1) then overwrites K(t-1), read in iteration
    // t-1; V(t+1) overwrites V(t-2), read in iteration t-1.
    v4u32 pprev[4];
    bool has_prev = false;  // wave-uniform: a P of an earlier tile awaits its product
    int vprev = 0;          // its V stage
    auto flush = [&]() {
        if (has_prev) pv_hd<DT, D>(vbuf[vprev], vo, pprev, oacc);
        has_prev = false;
    };
    auto step = [&](int t, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        if (SKEW)
            wait_vmcnt<NI>();  // this wave's K(t) (and V(t-1)) landed
        else
            wait_vmcnt<0>();   // this wave's loads of tile t landed
        __syncthreads();       // everyone's landed; the stages reloaded next are free
        if (t + 1 < n_tiles) issue(t + 1);
        if (EDGE && CAUSAL && t * BN > wq0 + 31) {  // no key visible
            if (SKEW) flush();
            return;
        }
        v16f32 s[2];
        v4u32 pf[4];
        qk_hd<DT, D>(kbuf[t & 1], ko, qf, s);
        if (SKEW) {
            auto pending = [&]() {
                flush();
                if (!EDGE) hd_sched_skewed<NO>();
            };
            softmax_tile<DT, CAUSAL, EDGE, NO>(s, pf, oacc, st, c, t * BN, T, my_q, hh, pending);
#pragma unroll
            for (int i = 0; i < 4; ++i) pprev[i] = pf[i];
            has_prev = true;
            vprev = t % kVStages;
        } else {
            softmax_tile<DT, CAUSAL, EDGE, NO>(s, pf, oacc, st, c, t * BN, T, my_q, hh);
            pv_hd<DT, D>(vbuf[t & 1], vo, pf, oacc);
        }
    };
    int t = 0;
    for (; t < n_main; ++t) step(t, std::integral_constant<bool, false>());
    for (; t < n_tiles; ++t) step(t, std::integral_constant<bool, true>());
    if (SKEW) {
        wait_vmcnt<0>();
        __syncthreads();  // every wave's loads of the last V tile landed
        flush();
    }

    const float lt = halves_sum(st.l);
    const float inv = 1.0f / lt;
    if (my_q < T) {
        uint16_t* orow = o + base + (int64_t)my_q * D;
#pragma unroll
        for (int mt = 0; mt < NO; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v2u32 w;
                w[0] = pack2<DT>(oacc[mt][4 * g] * inv, oacc[mt][4 * g + 1] * inv);
                w[1] = pack2<DT>(oacc[mt][4 * g + 2] * inv, oacc[mt][4 * g + 3] * inv);
                *(v2u32*)(orow + 32 * mt + acc_row(4 * g, hh)) = w;
            }
        if (lse != nullptr && hh == 0)
            lse[(int64_t)bh * T + my_q] = (st.mc + log2f(lt)) * kLn2;
    }
}

template <int DT, int D>
static const void* hd_ptr(bool causal) {
    return causal ? (const void*)fused_hd16<DT, true, D> : (const void*)fused_hd16<DT, false, D>;
}

hipError_t launch_fused_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int BH, int T, int D, int causal, float c, bool negate_q, int dt,
                           hipStream_t stream) {
    const int nq = (T + kBlockM - 1) / kBlockM;
    const dim3 grid((unsigned)(nq * BH));
    const dim3 block(kThreads);
    const uint32_t sign = negate_q ? 0x80008000u : 0u;
    const void* fn = hd_kernel_ptr(((D == 128) ? 4 : 0) + (dt == ATTN_DT_F16 ? 2 : 0) +
                                   (causal ? 0 : 1));
    if (fn == nullptr) return hipErrorInvalidValue;
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    uint16_t* oo = (uint16_t*)o;
    void* args[] = {&qq, &kk, &vv, &oo, &lse, &T, (void*)&nq, &c, (void*)&sign};
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

// Table order: D = 32 then 128; bf16 then f16; causal then not.
const void* hd_kernel_ptr(int index) {
    switch (index) {
        case 0: return hd_ptr<ATTN_DT_BF16, 32>(true);
        case 1: return hd_ptr<ATTN_DT_BF16, 32>(false);
        case 2: return hd_ptr<ATTN_DT_F16, 32>(true);
        case 3: return hd_ptr<ATTN_DT_F16, 32>(false);
        case 4: return hd_ptr<ATTN_DT_BF16, 128>(true);
        case 5: return hd_ptr<ATTN_DT_BF16, 128>(false);
        case 6: return hd_ptr<ATTN_DT_F16, 128>(true);
        case 7: return hd_ptr<ATTN_DT_F16, 128>(false);
        default: return nullptr;
    }
}

}  // namespace attn
