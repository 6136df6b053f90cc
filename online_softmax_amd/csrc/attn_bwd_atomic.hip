// The attention backward pass in one main kernel: each workgroup owns a
// block of keys, streams the query tiles that see it, and accumulates dK and
// dV in registers as the split backward's bwd_kv16 does, but also forms the
// block's share of dQ = scale dS K for every tile and adds it into a float32
// copy of dQ with atomic adds, so S and dP are computed once instead of twice.
//
// "Flash attention in PyTorch, then in Triton", section "Backwards, and
// training with it", defines the products (P made again from the scores and
// the saved log-sum-exp, dV = P^T dO, dP = dO V^T, dS = P (dP - delta),
// dQ = scale dS K, dK = scale dS^T Q) and notes that a key block's dQ
// contributions must be summed across blocks; here that sum is done by
// float32 atomics in HBM instead of a second pass.
//
// gfx950 design, three launches on one stream:
//  - bwd_prep16: -delta = -rowsum(dO * O) and a zero fill of the float32 dQ
//    copy (a kernel, not a memset, so the sequence can be captured in a graph).
//  - bwd_kvq16: 4 wave64s, 32 keys per wave, 128 per workgroup, query tiles of
//    64 through a 2-stage LDS ring loaded one tile ahead by direct buffer
//    loads. Per tile and 32-query half, each wave computes S and dP on the
//    matrix cores, P and dS on the vector ALU, and dV^T += dO^T P,
//    dK^T += Q^T dS; its packed dS goes to an LDS copy of dS^T (row = key).
//    After a barrier, wave w forms the 32 x 32 block (queries 32(w/2) ..,
//    dims 32(w%2) ..) of the tile's dQ over all 128 keys: A = dS read
//    transposed from that copy, B = the block's K, loaded into LDS once and
//    read transposed the same way. The 16 sums per lane go to dQ as global
//    float atomic adds at once; the wait for a later tile's loads counts
//    them (vector-memory operations complete in issue order) instead of
//    draining them.
//  - bwd_dq_finish16: dQ = scale * (the float32 copy), rounded to the dtype.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bwd_tiles.h"
#include "fused_layout.h"
#include "gfx950.h"
#include "kernels.h"

namespace attn {

namespace {
constexpr float kLog2eA = 1.4426950408889634074f;
}

// -delta (as bwd_delta16) and zeros for the float32 dQ rows: 8 lanes per
// row, 32 rows per workgroup.
template <int DT>
__global__ __launch_bounds__(256) void bwd_prep16(const uint16_t* __restrict__ o,
                                                  const uint16_t* __restrict__ dout,
                                                  float* __restrict__ ndelta,
                                                  float* __restrict__ dq_acc, int64_t rows) {
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
        const v4f32 z = {0.f, 0.f, 0.f, 0.f};
        *(v4f32*)(dq_acc + row * kHeadDim + 8 * part) = z;
        *(v4f32*)(dq_acc + row * kHeadDim + 8 * part + 4) = z;
    }
    acc += __shfl_xor(acc, 1, 8);
    acc += __shfl_xor(acc, 2, 8);
    acc += __shfl_xor(acc, 4, 8);
    if (row < rows && part == 0) ndelta[row] = -acc;
}

// dq = scale * dq_acc rounded to the dtype, 8 values per lane.
template <int DT>
__global__ __launch_bounds__(256) void bwd_dq_finish16(const float* __restrict__ dq_acc,
                                                       uint16_t* __restrict__ dq, int64_t n8,
                                                       float scale) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const v4f32 a = *(const v4f32*)(dq_acc + 8 * i);
    const v4f32 b = *(const v4f32*)(dq_acc + 8 * i + 4);
    v4u32 w;
    w[0] = pack2<DT>(a[0] * scale, a[1] * scale);
    w[1] = pack2<DT>(a[2] * scale, a[3] * scale);
    w[2] = pack2<DT>(b[0] * scale, b[1] * scale);
    w[3] = pack2<DT>(b[2] * scale, b[3] * scale);
    *(v4u32*)(dq + 8 * i) = w;
}

// ---------------------------------------------------------------------------
// dK, dV and the dQ sums. Workgroup: a block of kBwdBlockKV keys of one slice
// (bwd_kv_tile_of); query tiles of kBwdBlockQ from the first that sees the
// block (causal) to the last. c = |scale| log2(e); ksign negates the K rows
// of the scores for a negative scale; scale multiplies dK at the end (and dQ
// in bwd_dq_finish16).
// ---------------------------------------------------------------------------
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_kvq16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ ndelta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ dq_acc, int T,
    int nkb, float c, float scale, uint32_t ksign) {
    constexpr int kStages = 2;
    __shared__ __attribute__((aligned(1024))) char qring[kStages][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char dring[kStages][kTileBytes16];
    // dS^T of the block for the current query tile, and the block's K rows
    // (two 64-key tiles each, swz_b)
    __shared__ __attribute__((aligned(1024))) char sbuf[2][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char kbuf[2][kTileBytes16];
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
    const float kbias = CAUSAL || my_key < T ? 0.f : -INFINITY;

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

    const uint32_t slice_bytes = (uint32_t)T * (kHeadDim * 2);
    const v4u32_rsrc krs = buffer_rsrc(k + base, slice_bytes);
    const v4u32_rsrc qrs = buffer_rsrc(q + base, slice_bytes);
    const v4u32_rsrc drs = buffer_rsrc(dout + base, slice_bytes);
    const v4u32_rsrc lrs = buffer_rsrc(lse + (int64_t)bh * T, (uint32_t)T * 4u);
    const v4u32_rsrc ers = buffer_rsrc(ndelta + (int64_t)bh * T, (uint32_t)T * 4u);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[i] = (uint32_t)dlb_global_byte(wave, i, lane);

    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    const int t0 = bwd_first_qtile(kb, CAUSAL);
    const int n = nqt - t0;
    auto issue = [&](int u) {
        const int q0 = (t0 + u) * kBwdBlockQ;
        const int st = u % kStages;
        load_btile(qrs, voff, q0, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)qring[st]);
        load_btile(drs, voff, q0, T, wave_u, (uint32_t)(uintptr_t)(lds_void*)dring[st]);
        const uint32_t row = (uint32_t)min(q0 + lane, T - 1) * 4u;
        if (wave_u == 0) dma4(lrs, row, (uint32_t)(uintptr_t)(lds_void*)lring[st]);
        if (wave_u == 1) dma4(ers, row, (uint32_t)(uintptr_t)(lds_void*)ering[st]);
    };

    // lane bases of the fragment reads
    uint32_t rb[4], tb[2][2], tq[2], tk[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rb[ks] = (uint32_t)bfrag_byte(ql, hh, 0, ks);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) tb[ct][half] = (uint32_t)btr_byte(lane, ct, 0, half);
        tq[half] = (uint32_t)btr_byte(lane, bwd_dq_qhalf(wave), 0, half);
        tk[half] = (uint32_t)btr_byte(lane, bwd_dq_dhalf(wave), 0, half);
    }

    // The block's K rows (two 64-row tiles, rows past T clamped; their dS is
    // zero) and the first query tile.
#pragma unroll
    for (int i = 0; i < 2; ++i)
        load_btile(krs, voff, kb * kBwdBlockKV + 64 * i, T, wave_u,
                   (uint32_t)(uintptr_t)(lds_void*)kbuf[i]);
    if (n >= 1) issue(0);
    wait_vmcnt<0>();
    __syncthreads();

    v16f32 dkt[2], dvt[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkt[ct][r] = dvt[ct][r] = 0.f;

    auto rows4 = [&](const char* tile, int mt, v4u32(&f)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) f[ks] = brow_at(lane_tile(tile, rb[ks]), mt);
    };
    auto prod4 = [&](const v4u32(&f)[4], const v4u32(&bf)[4], v16f32& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16<DT>(f[ks], bf[ks], acc);
    };
    // P and dS of half mt of query tile u packed into the B operands of dV^T
    // and dK^T (as bwd_kv16). EDGE tiles mask query rows past T and (causal)
    // queries before the lane's key; the lane's queries are
    // q0 + 32mt + acc_row(r, hh). Non-causal, a key past T gets P = 0 on
    // every tile from a -inf bias in the exponent (causal, the tiles that
    // hold such keys are all EDGE tiles, whose mask covers them).
    auto make_pds = [&](int u, int mt, const v16f32& s, const v16f32& dp, v4u32(&pf)[2],
                        v4u32(&sf)[2], auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const int st = u % kStages;
        const int q0h = (t0 + u) * kBwdBlockQ + 4 * hh;
        const int room = T - q0h;
        const int lag = my_key - q0h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int qi0 = 32 * mt + 8 * g + 4 * hh;
            const v4f32 l4 = *(const v4f32*)&lring[st][qi0];
            float pv[4], dsv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                float p = fast_exp2(fmaf(s[r], c, fmaf(-l4[i], kLog2eA, kbias)));
                if (EDGE) {
                    const int off = 32 * mt + 8 * g + i;
                    p = (off < room && (!CAUSAL || off >= lag)) ? p : 0.f;
                }
                pv[i] = p;
                dsv[i] = p * dp[r];  // dp holds dP - delta
            }
            const int kl = g >> 1, w0 = 2 * (g & 1);
            pf[kl][w0] = pack2<DT>(pv[0], pv[1]);
            pf[kl][w0 + 1] = pack2<DT>(pv[2], pv[3]);
            sf[kl][w0] = pack2<DT>(dsv[0], dsv[1]);
            sf[kl][w0 + 1] = pack2<DT>(dsv[2], dsv[3]);
        }
    };
    char* const sflat = &sbuf[0][0];
    // one 32-query half of tile u: S, dP, P and dS, dV^T and dK^T, and the
    // packed dS into the wave's rows of dS^T
    auto half = [&](int u, int mt, auto edge_tag) {
        const int st = u % kStages;
        v16f32 s, dp;
        {
            v4u32 f[4];
            rows4(qring[st], mt, f);
            prod4(f, kf, s);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            // dP - delta: the accumulator starts from -delta of the half's
            // queries (register r: query 32mt + acc_row(r, hh))
            v4u32 f[4];
            rows4(dring[st], mt, f);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const v4f32 e4 = *(const v4f32*)&ering[st][32 * mt + 8 * g + 4 * hh];
#pragma unroll
                for (int i = 0; i < 4; ++i) dp[4 * g + i] = e4[i];
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) dp = mfma16<DT>(f[ks], vf[ks], dp);
        }
        __builtin_amdgcn_sched_barrier(0);
        v4u32 pf[2], sf[2];
        make_pds(u, mt, s, dp, pf, sf, edge_tag);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v2u32 w2 = {sf[g >> 1][2 * (g & 1)], sf[g >> 1][2 * (g & 1) + 1]};
            *(v2u32*)(sflat + bwd_ds_byte(wave, ql, hh, mt, g)) = w2;
        }
        __builtin_amdgcn_sched_barrier(0);
        const lds_char* dtr[2][2];
        const lds_char* qtr[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                dtr[ct][hf] = lane_tile(dring[st], tb[ct][hf]);
                qtr[ct][hf] = lane_tile(qring[st], tb[ct][hf]);
            }
#pragma unroll
        for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                dvt[ct] = mfma16<DT>(btr_at(dtr[ct][0], dtr[ct][1], 2 * mt + kl), pf[kl],
                                     dvt[ct]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                dkt[ct] = mfma16<DT>(btr_at(qtr[ct][0], qtr[ct][1], 2 * mt + kl), sf[kl],
                                     dkt[ct]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // zeros in the wave's 32 rows of dS^T (a tile the wave's keys do not see)
    auto zero_rows = [&]() {
        const v4u32 z = {0u, 0u, 0u, 0u};
        char* row = sflat + kTileBytes16 * (wave >> 1) + 128 * (32 * (wave & 1) + (lane >> 1)) +
                    64 * (lane & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) *(v4u32*)(row + 16 * i) = z;
    };
    // the wave's block of the tile's dQ over the block's 128 keys
    auto dq_product = [&](v16f32& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            acc = mfma16<DT>(btr(sbuf[ks >> 2], tq[0], tq[1], ks & 3),
                             btr(kbuf[ks >> 2], tk[0], tk[1], ks & 3), acc);
            if (ks == 3) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // add the block of tile u into dQ: lane (ql, hh) holds dim
    // 32 * dhalf + ql of queries 32 * qhalf + acc_row(r, hh). A query row
    // past T holds an exact zero (its P and dS are masked), so it is added
    // to row T - 1 instead: every lane issues all 16 atomics, which keeps
    // the count of vector-memory operations per tile fixed.
    float* const dq_lane = dq_acc + base + 32 * bwd_dq_dhalf(wave) + ql;
    auto flush = [&](int u, const v16f32& acc) {
        const int qb = (t0 + u) * kBwdBlockQ + 32 * bwd_dq_qhalf(wave);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = min(qb + acc_row(r, hh), T - 1);
            unsafeAtomicAdd(dq_lane + (int64_t)row * kHeadDim, acc[r]);
        }
    };

    using Y = std::integral_constant<bool, true>;
    using N = std::integral_constant<bool, false>;
    // Tile u: wait for its loads (issued one tile ahead), a barrier (every
    // wave is done with tile u - 1: its ring stage and dS^T are free), the
    // loads of tile u + 1; the wave's half-tiles (or zeros); a barrier; the
    // dQ product and its 16 atomics. Vector-memory operations complete in
    // issue order, so the wait lets tile u - 1's 16 atomics stay in flight.
    auto top = [&](int u) {
        if (u > 0) {
            wait_vmcnt<16>();
            __syncthreads();
        }
        if (u + 1 < n) issue(u + 1);
    };
    auto bottom = [&](int u) {
        __syncthreads();
        v16f32 acc;
        dq_product(acc);
        flush(u, acc);
    };
    const int uw = bwd_kv_first_seen(kb, wave_u, n, CAUSAL);
    int u = 0;
    for (; u < uw && u < n; ++u) {
        top(u);
        zero_rows();
        bottom(u);
    }
    if (u < n) {
        // the wave's first tile takes the masked form (the causal diagonal)
        top(u);
        half(u, 0, Y());
        half(u, 1, Y());
        bottom(u);
        ++u;
        for (; u + 1 < n; ++u) {
            top(u);
            half(u, 0, N());
            half(u, 1, N());
            bottom(u);
        }
        if (u < n) {
            top(u);
            if (bwd_kv_edge(kb, wave_u, u, T, CAUSAL)) {
                half(u, 0, Y());
                half(u, 1, Y());
            } else {
                half(u, 0, N());
                half(u, 1, N());
            }
            bottom(u);
            ++u;
        }
    }
    if (my_key < T) {
        store_rows<DT>(dk + base + (int64_t)my_key * kHeadDim, dkt, scale, hh);
        store_rows<DT>(dv + base + (int64_t)my_key * kHeadDim, dvt, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
// Launcher and kernel table.
// ---------------------------------------------------------------------------
hipError_t launch_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, float* dq_acc, int BH, int T, int causal, float c,
                             float scale, bool negate, int dt, hipStream_t stream) {
    const uint32_t sign = negate ? 0x80008000u : 0u;
    const int64_t rows = (int64_t)BH * T;
    const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
    const dim3 block(kThreads);
    const uint16_t* q16 = (const uint16_t*)q;
    const uint16_t* k16 = (const uint16_t*)k;
    const uint16_t* v16 = (const uint16_t*)v;
    const uint16_t* o16 = (const uint16_t*)o;
    const uint16_t* d16 = (const uint16_t*)dout;
    const dim3 prep_grid((unsigned)((rows + 31) / 32));
    const int64_t n8 = rows * (kHeadDim / 8);
    const dim3 fin_grid((unsigned)((n8 + 255) / 256));
    if (dt == ATTN_DT_BF16) {
        hipLaunchKernelGGL(bwd_prep16<ATTN_DT_BF16>, prep_grid, dim3(256), 0, stream, o16, d16,
                           delta, dq_acc, rows);
        auto kvq = causal ? bwd_kvq16<ATTN_DT_BF16, true> : bwd_kvq16<ATTN_DT_BF16, false>;
        hipLaunchKernelGGL(kvq, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dk, (uint16_t*)dv, dq_acc, T, nkb, c,
                           scale, sign);
        hipLaunchKernelGGL(bwd_dq_finish16<ATTN_DT_BF16>, fin_grid, dim3(256), 0, stream,
                           dq_acc, (uint16_t*)dq, n8, scale);
    } else {
        hipLaunchKernelGGL(bwd_prep16<ATTN_DT_F16>, prep_grid, dim3(256), 0, stream, o16, d16,
                           delta, dq_acc, rows);
        auto kvq = causal ? bwd_kvq16<ATTN_DT_F16, true> : bwd_kvq16<ATTN_DT_F16, false>;
        hipLaunchKernelGGL(kvq, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse, delta, (uint16_t*)dk, (uint16_t*)dv, dq_acc, T, nkb, c,
                           scale, sign);
        hipLaunchKernelGGL(bwd_dq_finish16<ATTN_DT_F16>, fin_grid, dim3(256), 0, stream,
                           dq_acc, (uint16_t*)dq, n8, scale);
    }
    return hipGetLastError();
}

const void* bwd_atomic_kernel_ptr(int index) {
    switch (index) {
        case 0: return (const void*)bwd_prep16<ATTN_DT_BF16>;
        case 1: return (const void*)bwd_kvq16<ATTN_DT_BF16, true>;
        case 2: return (const void*)bwd_kvq16<ATTN_DT_BF16, false>;
        case 3: return (const void*)bwd_dq_finish16<ATTN_DT_BF16>;
        case 4: return (const void*)bwd_prep16<ATTN_DT_F16>;
        case 5: return (const void*)bwd_kvq16<ATTN_DT_F16, true>;
        case 6: return (const void*)bwd_kvq16<ATTN_DT_F16, false>;
        case 7: return (const void*)bwd_dq_finish16<ATTN_DT_F16>;
        default: return nullptr;
    }
}

}  // namespace attn
