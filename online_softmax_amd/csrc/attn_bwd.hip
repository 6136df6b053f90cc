// The attention backward pass for gfx950: dQ, dK and dV from the output
// gradient dO, the forward's output O and its per-row log-sum-exp.
//
// "Flash attention in PyTorch, then in Triton", section "Backwards, and
// training with it", defines the pass: the probabilities are made again
// from the scores and the saved log-sum-exp, P = exp(s - lse); dV = P^T dO;
// dP = dO V^T; the softmax's backward gives dS = P (dP - delta) with delta
// each row's sum of dO * O, computed once; dQ = scale dS K and dK = scale
// dS^T Q. The work is split into two kernels so that no two workgroups write
// one place: bwd_kv16 owns a block of keys and streams the query tiles that
// see them (dK, dV), bwd_q16 owns a block of queries and streams the key
// tiles they see (dQ). Both recompute S and dP; accumulators are float32.
//
// gfx950 design (the page's kernels are Triton programs for an RTX 4090):
//  - bwd_kv16: 4 wave64s, 32 keys per wave (128 per workgroup); the wave's K
//    and V rows stay in VGPRs as the B operands of S = Q K^T and
//    dP = dO V^T, so one lane owns one key and 16 of the 32 query rows of an
//    MFMA tile. P and dS, packed to 16-bit from those accumulators, are the
//    B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands are
//    transposed LDS reads (ds_read_b64_tr_b16) of the same Q and dO tiles.
//  - bwd_q16: 4 wave64s, 32 queries per wave; Q and dO rows in VGPRs,
//    S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T with K^T read
//    transposed from the K tile. lse and delta are per-lane scalars.
//  - Tiles of 64 rows x 128 bytes arrive by direct buffer loads into a
//    3-stage LDS ring, two tiles ahead, in the swizzle swz_b (fused_layout.h)
//    that keeps both the row and the transposed fragment reads free of bank
//    conflicts.
//  - Masks: causal (key after query), and query rows past T in bwd_kv16 (key
//    rows past T in bwd_q16); masked P and dS are set to 0 by selection, so
//    no clamped or stale value can reach a sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fused_layout.h"
#include "gfx950.h"
#include "kernels.h"

namespace attn {

constexpr float kLog2e = 1.4426950408889634074f;

// delta_i = sum_e dO[i,e] * O[i,e] in float32, 8 lanes per row (one 16-byte
// chunk of 8 16-bit values each), reduced across the 8 lanes.
template <int DT>
__global__ __launch_bounds__(256) void bwd_delta16(const uint16_t* __restrict__ o,
                                                   const uint16_t* __restrict__ dout,
                                                   float* __restrict__ delta,
                                                   int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    float acc = 0.f;
    if (row < rows) {
        const v4u32 a = *(const v4u32*)(o + row * kHeadDim + 8 * part);
        const v4u32 b = *(const v4u32*)(dout + row * kHeadDim + 8 * part);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(lo16<DT>(a[i]), lo16<DT>(b[i]), acc);
            acc = fmaf(hi16<DT>(a[i]), hi16<DT>(b[i]), acc);
        }
    }
    acc += __shfl_xor(acc, 1, 8);
    acc += __shfl_xor(acc, 2, 8);
    acc += __shfl_xor(acc, 4, 8);
    if (row < rows && part == 0) delta[row] = acc;
}

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

// ---------------------------------------------------------------------------
// dK and dV. Workgroup: a block of kBwdBlockKV keys of one slice; query tiles
// of kBwdBlockQ stream through the ring from the first one that sees the
// block (causal) to the last. c = |scale| log2(e); ksign negates K for a
// negative scale; scale multiplies dK at the end.
// ---------------------------------------------------------------------------
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_kv16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int T, int nkb, float c,
    float scale, uint32_t ksign) {
    constexpr int kStages = 3;
    __shared__ __attribute__((aligned(1024))) char qring[kStages][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char dring[kStages][kTileBytes16];
    __shared__ __attribute__((aligned(256))) float lring[kStages][kBwdBlockQ];
    __shared__ __attribute__((aligned(256))) float ering[kStages][kBwdBlockQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, kb;
    bwd_kv_tile_of(blockIdx.x, gridDim.x, nkb, CAUSAL, &bh, &kb);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const int kw0 = kb * kBwdBlockKV + 32 * wave;  // first key of this wave
    const int my_key = kw0 + ql;                   // this lane's key

    // K and V rows of the lane's key: B operands of S = Q K^T and dP = dO V^T
    v4u32 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (my_key < T) {
            x = *(const v4u32*)(k + base + (int64_t)my_key * kHeadDim + q_col16(hh, ks));
            y = *(const v4u32*)(v + base + (int64_t)my_key * kHeadDim + q_col16(hh, ks));
        }
        kf[ks] = x ^ ksign;
        vf[ks] = y;
    }
    wait_vmcnt<0>();

    const uint32_t slice_bytes = (uint32_t)T * (kHeadDim * 2);
    const v4u32_rsrc qrs = buffer_rsrc(q + base, slice_bytes);
    const v4u32_rsrc drs = buffer_rsrc(dout + base, slice_bytes);
    const v4u32_rsrc lrs = buffer_rsrc(lse + (int64_t)bh * T, (uint32_t)T * 4u);
    const v4u32_rsrc ers = buffer_rsrc(delta + (int64_t)bh * T, (uint32_t)T * 4u);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[i] = (uint32_t)dlb_global_byte(wave, i, lane);

    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    const int t0 = bwd_first_qtile(kb, CAUSAL);
    const int n = nqt - t0;
    // loads of tile u: Q and dO (2 each per wave); lse by wave 0, delta by
    // wave 1 (one 4-byte-per-lane load each)
    const int per_tile = 4 + (wave_u < 2 ? 1 : 0);
    auto issue = [&](int u) {
        const int q0 = (t0 + u) * kBwdBlockQ;
        const int st = u % kStages;
        load_btile(qrs, voff, q0, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)qring[st]);
        load_btile(drs, voff, q0, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)dring[st]);
        const uint32_t row = (uint32_t)min(q0 + lane, T - 1) * 4u;
        if (wave_u == 0) dma4(lrs, row, (uint32_t)(uintptr_t)(lds_void*)lring[st]);
        if (wave_u == 1) dma4(ers, row, (uint32_t)(uintptr_t)(lds_void*)ering[st]);
    };

    // lane bases of the fragment reads (shared by the Q and dO tiles)
    uint32_t rb[4], tb[2][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rb[ks] = (uint32_t)bfrag_byte(ql, hh, 0, ks);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int half = 0; half < 2; ++half) tb[ct][half] = (uint32_t)btr_byte(lane, ct, 0, half);

    v16f32 dkt[2], dvt[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkt[ct][r] = dvt[ct][r] = 0.f;

    if (n >= 1) issue(0);
    if (n >= 2) issue(1);
    for (int u = 0; u < n; ++u) {
        // tile u landed for this wave (tile u+1 may still be in flight)
        if (u + 1 < n) {
            if (per_tile == 5) wait_vmcnt<5>(); else wait_vmcnt<4>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        if (u + 2 < n) issue(u + 2);
        const int qt = t0 + u;
        const int q0 = qt * kBwdBlockQ;
        if (CAUSAL && q0 + kBwdBlockQ - 1 < kw0) continue;  // the wave's keys see none
        const int st = u % kStages;
        const char* qt_ = qring[st];
        const char* dt_ = dring[st];
        v16f32 s[2], dp[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mt][r] = dp[mt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = mfma16<DT>(brow(qt_, rb[ks], mt), kf[ks], s[mt]);
                dp[mt] = mfma16<DT>(brow(dt_, rb[ks], mt), vf[ks], dp[mt]);
            }
        // P and dS; the lane's queries are q0 + 32mt + acc_row(r, hh)
        v4u32 pf[4], sf[4];
        const bool edge = (CAUSAL && q0 < kw0 + 31) || q0 + kBwdBlockQ > T;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qi0 = 32 * mt + 8 * g + 4 * hh;  // 4 consecutive queries
                const v4f32 l4 = *(const v4f32*)&lring[st][qi0];
                const v4f32 e4 = *(const v4f32*)&ering[st][qi0];
                float pv[4], dsv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;
                    float p = fast_exp2(fmaf(s[mt][r], c, -l4[i] * kLog2e));
                    float d = p * (dp[mt][r] - e4[i]);
                    if (edge) {
                        const int qi = q0 + qi0 + i;
                        const bool keep = qi < T && (!CAUSAL || my_key <= qi);
                        p = keep ? p : 0.f;
                        d = keep ? d : 0.f;
                    }
                    pv[i] = p;
                    dsv[i] = d;
                }
                // registers r = 4g..4g+3 of half-tile mt belong to step
                // ks = 2mt + g/2, dwords 2(g&1), 2(g&1)+1
                const int ks = 2 * mt + (g >> 1), w0 = 2 * (g & 1);
                pf[ks][w0] = pack2<DT>(pv[0], pv[1]);
                pf[ks][w0 + 1] = pack2<DT>(pv[2], pv[3]);
                sf[ks][w0] = pack2<DT>(dsv[0], dsv[1]);
                sf[ks][w0 + 1] = pack2<DT>(dsv[2], dsv[3]);
            }
        // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                dvt[ct] = mfma16<DT>(btr(dt_, tb[ct][0], tb[ct][1], ks), pf[ks], dvt[ct]);
                dkt[ct] = mfma16<DT>(btr(qt_, tb[ct][0], tb[ct][1], ks), sf[ks], dkt[ct]);
            }
    }
    if (my_key < T) {
        store_rows<DT>(dk + base + (int64_t)my_key * kHeadDim, dkt, scale, hh);
        store_rows<DT>(dv + base + (int64_t)my_key * kHeadDim, dvt, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
// dQ. Workgroup: kBlockM queries of one slice (tile_of, as the forward);
// key tiles stream through the ring up to the block's last query (causal).
// qsign negates Q for a negative scale; scale multiplies dQ at the end.
// ---------------------------------------------------------------------------
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_q16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int T, int nq, float c, float scale, uint32_t qsign) {
    constexpr int kStages = 3;
    constexpr int BN = kBlockN16;
    __shared__ __attribute__((aligned(1024))) char kring[kStages][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char vring[kStages][kTileBytes16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const int wq0 = qt * kBlockM + 32 * wave;
    const int my_q = wq0 + ql;

    v4u32 qf[4], of[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (my_q < T) {
            x = *(const v4u32*)(q + base + (int64_t)my_q * kHeadDim + q_col16(hh, ks));
            y = *(const v4u32*)(dout + base + (int64_t)my_q * kHeadDim + q_col16(hh, ks));
        }
        qf[ks] = x ^ qsign;
        of[ks] = y;
    }
    float lse2 = 0.f, dl = 0.f;
    if (my_q < T) {
        lse2 = lse[(int64_t)bh * T + my_q] * kLog2e;
        dl = delta[(int64_t)bh * T + my_q];
    }
    wait_vmcnt<0>();

    const uint32_t slice_bytes = (uint32_t)T * (kHeadDim * 2);
    const v4u32_rsrc krs = buffer_rsrc(k + base, slice_bytes);
    const v4u32_rsrc vrs = buffer_rsrc(v + base, slice_bytes);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[i] = (uint32_t)dlb_global_byte(wave, i, lane);
    const int n = key_tiles(qt, T, BN, CAUSAL);
    auto issue = [&](int u) {
        const int st = u % kStages;
        load_btile(krs, voff, u * BN, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)kring[st]);
        load_btile(vrs, voff, u * BN, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)vring[st]);
    };

    uint32_t rb[4], tb[2][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rb[ks] = (uint32_t)bfrag_byte(ql, hh, 0, ks);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int half = 0; half < 2; ++half) tb[ct][half] = (uint32_t)btr_byte(lane, ct, 0, half);

    v16f32 dqt[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[ct][r] = 0.f;

    if (n >= 1) issue(0);
    if (n >= 2) issue(1);
    for (int u = 0; u < n; ++u) {
        if (u + 1 < n)
            wait_vmcnt<4>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (u + 2 < n) issue(u + 2);
        const int k0 = u * BN;
        if (CAUSAL && k0 > wq0 + 31) continue;  // no key of the tile is visible
        const int st = u % kStages;
        const char* kt_ = kring[st];
        const char* vt_ = vring[st];
        v16f32 s[2], dp[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[nt][r] = dp[nt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                s[nt] = mfma16<DT>(brow(kt_, rb[ks], nt), qf[ks], s[nt]);
                dp[nt] = mfma16<DT>(brow(vt_, rb[ks], nt), of[ks], dp[nt]);
            }
        // dS^T; the lane's keys are k0 + 32nt + acc_row(r, hh)
        v4u32 sf[4];
        const bool edge = (CAUSAL && k0 + BN - 1 > wq0) || k0 + BN > T;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int nt = ks >> 1, r0 = (ks & 1) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = r0 + 2 * i + e;
                    const float p = fast_exp2(fmaf(s[nt][r], c, -lse2));
                    float d = p * (dp[nt][r] - dl);
                    if (edge) {
                        const int key = k0 + 32 * nt + acc_row(r, hh);
                        const bool keep = key < T && (!CAUSAL || key <= my_q);
                        d = keep ? d : 0.f;
                    }
                    d2[e] = d;
                }
                sf[ks][i] = pack2<DT>(d2[0], d2[1]);
            }
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                dqt[ct] = mfma16<DT>(btr(kt_, tb[ct][0], tb[ct][1], ks), sf[ks], dqt[ct]);
    }
    if (my_q < T) store_rows<DT>(dq + base + (int64_t)my_q * kHeadDim, dqt, scale, hh);
}

// ---------------------------------------------------------------------------
// Launcher and kernel table.
// ---------------------------------------------------------------------------
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, int BH, int T, int causal, float c, float scale,
                      bool negate, int dt, hipStream_t stream) {
    const uint32_t sign = negate ? 0x80008000u : 0u;
    const int64_t rows = (int64_t)BH * T;
    const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
    const int nq = (T + kBlockM - 1) / kBlockM;
    const dim3 block(kThreads);
    const uint16_t* q16 = (const uint16_t*)q;
    const uint16_t* k16 = (const uint16_t*)k;
    const uint16_t* v16 = (const uint16_t*)v;
    const uint16_t* o16 = (const uint16_t*)o;
    const uint16_t* d16 = (const uint16_t*)dout;
    if (dt == ATTN_DT_BF16) {
        hipLaunchKernelGGL(bwd_delta16<ATTN_DT_BF16>, dim3((unsigned)((rows + 31) / 32)),
                           dim3(256), 0, stream, o16, d16, delta, rows);
        auto kv = causal ? bwd_kv16<ATTN_DT_BF16, true> : bwd_kv16<ATTN_DT_BF16, false>;
        hipLaunchKernelGGL(kv, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dk, (uint16_t*)dv, T, nkb, c, scale,
                           sign);
        auto qk = causal ? bwd_q16<ATTN_DT_BF16, true> : bwd_q16<ATTN_DT_BF16, false>;
        hipLaunchKernelGGL(qk, dim3((unsigned)(nq * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dq, T, nq, c, scale, sign);
    } else {
        hipLaunchKernelGGL(bwd_delta16<ATTN_DT_F16>, dim3((unsigned)((rows + 31) / 32)),
                           dim3(256), 0, stream, o16, d16, delta, rows);
        auto kv = causal ? bwd_kv16<ATTN_DT_F16, true> : bwd_kv16<ATTN_DT_F16, false>;
        hipLaunchKernelGGL(kv, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dk, (uint16_t*)dv, T, nkb, c, scale,
                           sign);
        auto qk = causal ? bwd_q16<ATTN_DT_F16, true> : bwd_q16<ATTN_DT_F16, false>;
        hipLaunchKernelGGL(qk, dim3((unsigned)(nq * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dq, T, nq, c, scale, sign);
    }
    return hipGetLastError();
}

const void* bwd_kernel_ptr(int index) {
    switch (index) {
        case 0: return (const void*)bwd_delta16<ATTN_DT_BF16>;
        case 1: return (const void*)bwd_kv16<ATTN_DT_BF16, true>;
        case 2: return (const void*)bwd_kv16<ATTN_DT_BF16, false>;
        case 3: return (const void*)bwd_q16<ATTN_DT_BF16, true>;
        case 4: return (const void*)bwd_q16<ATTN_DT_BF16, false>;
        case 5: return (const void*)bwd_delta16<ATTN_DT_F16>;
        case 6: return (const void*)bwd_kv16<ATTN_DT_F16, true>;
        case 7: return (const void*)bwd_kv16<ATTN_DT_F16, false>;
        case 8: return (const void*)bwd_q16<ATTN_DT_F16, true>;
        case 9: return (const void*)bwd_q16<ATTN_DT_F16, false>;
        default: return nullptr;
    }
}

}  // namespace attn
