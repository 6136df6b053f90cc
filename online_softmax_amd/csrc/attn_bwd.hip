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
//  - Both kernels are software-pipelined on half-tiles of 32 rows: while the
//    vector ALU makes P and dS of one half (from the S the previous half
//    computed), the matrix cores compute dP of that half and S of the next,
//    then the half's gradient products run. The half-tile keeps the
//    pipeline's state within 256 VGPRs, so two workgroups share a CU.
//  - Masks: causal (key after query), and query rows past T in bwd_kv16 (key
//    rows past T in bwd_q16); masked P and dS are set to 0 by selection, so
//    no clamped or stale value can reach a sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bwd_tiles.h"
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
                                                   const float* __restrict__ lse,
                                                   float* __restrict__ ndelta,
                                                   float* __restrict__ lse2, int64_t rows) {
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
    if (row < rows && part == 0) {
        ndelta[row] = -acc;
        lse2[row] = lse[row] * kLog2e;
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
    const float* __restrict__ lse2, const float* __restrict__ ndelta,
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
    const v4u32_rsrc lrs = buffer_rsrc(lse2 + (int64_t)bh * T, (uint32_t)T * 4u);
    const v4u32_rsrc ers = buffer_rsrc(ndelta + (int64_t)bh * T, (uint32_t)T * 4u);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[i] = (uint32_t)dlb_global_byte(wave, i, lane);

    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    const int t0 = bwd_first_qtile(kb, CAUSAL);
    const int n = nqt - t0;
    // loads of tile u: Q and dO (2 each per wave); lse * log2(e) by wave 0,
    // -delta by wave 1 (one 4-byte-per-lane load each)
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

    // The pipeline runs on half-tiles of 32 queries (h = 2u + mt: rows
    // 32mt .. 32mt + 31 of query tile u), so its state (S of two halves,
    // dP, packed P and dS of one, their fragments) fits beside the
    // accumulators at two workgroups per CU.
    // Row fragments (A operands) of half mt of a Q or dO tile.
    auto rows4 = [&](const char* tile, int mt, v4u32(&f)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) f[ks] = brow_at(lane_tile(tile, rb[ks]), mt);
    };
    // acc = X B for 4 steps (X fragments f, B the lane's K or V row)
    auto prod4 = [&](const v4u32(&f)[4], const v4u32(&bf)[4], v16f32& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16<DT>(f[ks], bf[ks], acc);
    };
    // dP - delta of half mt of tile u: the accumulator starts from -delta of
    // the half's queries (register r: query 32mt + acc_row(r, hh)), so the
    // products leave dP - delta without a subtraction per score
    auto dp_minus_delta = [&](int u, int mt, const v4u32(&f)[4], v16f32& acc) {
        const int st = u % kStages;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v4f32 e4 = *(const v4f32*)&ering[st][32 * mt + 8 * g + 4 * hh];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * g + i] = e4[i];
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16<DT>(f[ks], vf[ks], acc);
    };
    // P and dS = P (dP - delta) of half mt of query tile u (dp holds dP -
    // delta), P = exp2(s c - lse log2 e) made again, packed into the B
    // operands of dV^T and dK^T
    // (steps 2mt, 2mt + 1). EDGE tiles mask query rows past T and (causal)
    // queries before the lane's key; the lane's queries are
    // q0 + 32mt + acc_row(r, hh).
    auto make_pds = [&](int u, int mt, const v16f32& s, const v16f32& dp, v4u32(&pf)[2],
                        v4u32(&sf)[2], auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const int st = u % kStages;
        // query q0 + 32mt + 8g + 4hh + i is kept when it is below T and
        // (causal) not before the lane's key: both tests against per-lane
        // bases with the constant 32mt + 8g + i
        const int q0h = (t0 + u) * kBwdBlockQ + 4 * hh;
        const int room = T - q0h;         // keep while offset < room
        const int lag = my_key - q0h;     // causal: keep while offset >= lag
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int qi0 = 32 * mt + 8 * g + 4 * hh;  // 4 consecutive queries
            const v4f32 l4 = *(const v4f32*)&lring[st][qi0];
            float pv[4], dsv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                float p = fast_exp2(fmaf(s[r], c, -l4[i]));
                if (EDGE) {  // a masked p is 0, so its dS is too
                    const int off = 32 * mt + 8 * g + i;
                    p = (off < room && (!CAUSAL || off >= lag)) ? p : 0.f;
                }
                pv[i] = p;
                dsv[i] = p * dp[r];
            }
            // registers r = 4g..4g+3 belong to step 2mt + g/2, dwords
            // 2(g&1), 2(g&1)+1
            const int kl = g >> 1, w0 = 2 * (g & 1);
            pf[kl][w0] = pack2<DT>(pv[0], pv[1]);
            pf[kl][w0 + 1] = pack2<DT>(pv[2], pv[3]);
            sf[kl][w0] = pack2<DT>(dsv[0], dsv[1]);
            sf[kl][w0 + 1] = pack2<DT>(dsv[2], dsv[3]);
        }
    };

    // Software pipeline over the half-tiles the wave sees: half h computes
    // dP of half h and S of half h + 1 on the matrix cores while the vector
    // ALU makes P and dS of half h (whose S the previous half produced),
    // then dV^T += dO^T P and dK^T += Q^T dS over the half's 32 queries.
    // Loads run two tiles ahead: at the top of tile u every load so far has
    // landed (tile u + 1, whose first half the second half of tile u needs),
    // and the barrier frees for tile u + 2 the stage tile u - 1 used.
    // First tile the wave sees (causal: the block's first query tile ends
    // before the keys of waves 2 and 3), from the wave-uniform copy of the
    // wave index, so the loop counter and the load offsets stay scalar.
    const int uw = bwd_kv_first_seen(kb, wave_u, n, CAUSAL);
    auto edge_of = [&](int u) { return bwd_kv_edge(kb, wave_u, u, T, CAUSAL); };
    using Y = std::integral_constant<bool, true>;
    using N = std::integral_constant<bool, false>;
    // SELF: the half computes its own S first (no overlap; the masked edge
    // tiles, which need more registers, run this way)
    auto half = [&](int u, int mt, v16f32& scur, v16f32& snext, auto next_tag, auto edge_tag,
                    auto self_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool SELF = decltype(self_tag)::value;
        const int st = u % kStages;
        if (SELF) {
            v4u32 f[4];
            rows4(qring[st], mt, f);
            prod4(f, kf, scur);
        }
        // the dO fragments, then (once the dP products hold them) the Q
        // fragments of the next half: the two sets are never live together
        v4u32 fd[4], fs[4];
        rows4(dring[st], mt, fd);
        __builtin_amdgcn_sched_barrier(0);
        v16f32 dp;
        v4u32 pf[2], sf[2];
        dp_minus_delta(u, mt, fd, dp);
        if (NEXT) {
            if (mt == 0)
                rows4(qring[st], 1, fs);
            else
                rows4(qring[(u + 1) % kStages], 0, fs);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (NEXT) prod4(fs, kf, snext);
        make_pds(u, mt, scur, dp, pf, sf, edge_tag);
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
    };
    // a pipelined tile (S of its first half already in sa; leaves S of the
    // next tile's first half in sa when NEXT)
    auto tile = [&](int u, v16f32& sa, v16f32& sb, auto next_tag) {
        half(u, 0, sa, sb, Y(), N(), N());
        half(u, 1, sb, sa, next_tag, N(), N());
    };
    // a masked tile, each half on its own
    auto edge_tile = [&](int u, v16f32& sa) {
        half(u, 0, sa, sa, N(), Y(), Y());
        half(u, 1, sa, sa, N(), Y(), Y());
    };
    auto sync_issue = [&](int u) {
        if (u > 0) {
            wait_vmcnt<0>();
            __syncthreads();
        }
        if (u + 2 < n) issue(u + 2);
    };

    if (n >= 1) issue(0);
    if (n >= 2) issue(1);
    wait_vmcnt<0>();
    __syncthreads();
    int u = 0;
    for (; u < uw && u < n; ++u) sync_issue(u);  // tiles the wave does not see
    if (u < n) {
        v16f32 sa, sb;
        // Only the wave's first tile can hold the causal diagonal and only
        // the slice's last tile can be ragged (bwd_kv_edge in
        // fused_layout.h; the host check walks every block, wave and
        // length), so the pipelined loop between them runs without masks.
        // The first tile always takes the masked form.
        sync_issue(u);
        edge_tile(u, sa);
        ++u;
        if (u < n) {
            // S of the first half of tile u: its stage landed at the last
            // wait
            {
                v4u32 f[4];
                rows4(qring[u % kStages], 0, f);
                prod4(f, kf, sa);
            }
            for (; u + 1 < n; ++u) {
                sync_issue(u);
                tile(u, sa, sb, Y());
            }
            sync_issue(u);
            if (edge_of(u))
                edge_tile(u, sa);
            else
                tile(u, sa, sb, N());
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
__global__ __launch_bounds__(kThreads, 3) void bwd_q16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ ndelta,
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
    float lq = 0.f, dl = 0.f;  // lse log2(e) and delta of the lane's query
    if (my_q < T) {
        lq = lse2[(int64_t)bh * T + my_q];
        dl = -ndelta[(int64_t)bh * T + my_q];
    }
    wait_vmcnt<0>();
    // -delta in every register: the start of each dP^T accumulator, so the
    // products leave dP - delta with no subtraction per score
    v16f32 ndl16;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndl16[r] = -dl;

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

    const uint32_t rb0 = (uint32_t)bfrag_byte(ql, hh, 0, 0);
    const uint32_t tb00 = (uint32_t)btr_byte(lane, 0, 0, 0);

    v16f32 dqt[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[ct][r] = 0.f;

    // The pipeline runs on half-tiles of 32 keys (h = 2u + nt: keys
    // k0 + 32nt .. k0 + 32nt + 31 of key tile u), so its state (S^T of two
    // halves, dP^T, packed dS^T of one, their fragments) fits beside the
    // accumulators at two workgroups per CU.
    // Row fragments (A operands) of half nt of a K or V tile.
    // (step ks's lane base is step 0's with bits 5-6 flipped by ks: the
    // swizzle permutes 32-byte pairs within a row, and ring stages are
    // 1024-aligned, so the flip commutes with adding the stage)
    auto rows4 = [&](const char* tile, int nt, v4u32(&f)[4]) {
        const uint32_t a0 = (uint32_t)(uintptr_t)lane_tile(tile, rb0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            f[ks] = brow_at((const lds_char*)(uintptr_t)(a0 ^ ((uint32_t)ks << 5)), nt);
    };
    // acc = X B for 4 steps (X fragments f, B the lane's Q or dO row)
    auto prod4 = [&](const v4u32(&f)[4], const v4u32(&bf)[4], v16f32& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16<DT>(f[ks], bf[ks], acc);
    };
    // dS^T = P (dP - delta) of half nt of key tile u, with P = exp2(s c -
    // lq) made again, packed into the B operands of dQ^T (steps 2nt,
    // 2nt + 1). EDGE tiles mask keys past T and (causal) keys after the
    // lane's query; the lane's keys are k0 + 32nt + acc_row(r, hh).
    auto make_ds = [&](int u, int nt, const v16f32& s, const v16f32& dp, v4u32(&sf)[2],
                       auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const int k0 = u * BN + 32 * nt;
#pragma unroll
        for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 8 * kl + 2 * i + e;
                    float p = fast_exp2(fmaf(s[r], c, -lq));
                    if (EDGE) {
                        const int key = k0 + acc_row(r, hh);
                        p = (key < T && (!CAUSAL || key <= my_q)) ? p : 0.f;
                    }
                    d[e] = p * dp[r];
                }
                sf[kl][i] = pack2<DT>(d[0], d[1]);
            }
    };

    // Software pipeline over the half-tiles the wave sees: half h computes
    // dP^T of half h and S^T of half h + 1 on the matrix cores while the
    // vector ALU makes P and dS of half h (whose S^T the previous half
    // produced), then dQ^T += K^T dS^T over the half's 32 keys. Loads run two
    // tiles ahead: at the top of tile u every load so far has landed (tile
    // u + 1, whose first half the second half of tile u needs), and the
    // barrier frees for tile u + 2 the stage tile u - 1 used.
    // The wave's last tile (causal: tiles past its last query are skipped),
    // from the wave-uniform copy of the wave index, so the loop counter and
    // the load offsets stay scalar.
    const int nw = bwd_q_tiles_seen(qt, wave_u, n, CAUSAL);
    using Y = std::integral_constant<bool, true>;
    using N = std::integral_constant<bool, false>;
    auto half = [&](int u, int nt, v16f32& scur, v16f32& snext, auto next_tag, auto edge_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int st = u % kStages;
        // the V fragments, then (once the dP products hold them) the K
        // fragments of the next half: the two sets are never live together
        v4u32 fd[4], fs[4];
        rows4(vring[st], nt, fd);
        __builtin_amdgcn_sched_barrier(0);
        v16f32 dp = ndl16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) dp = mfma16<DT>(fd[ks], of[ks], dp);
        if (NEXT) {
            if (nt == 0)
                rows4(kring[st], 1, fs);
            else
                rows4(kring[(u + 1) % kStages], 0, fs);
        }
        __builtin_amdgcn_sched_barrier(0);
        v4u32 sf[2];
        if (NEXT) prod4(fs, qf, snext);
        make_ds(u, nt, scur, dp, sf, edge_tag);
        __builtin_amdgcn_sched_barrier(0);
        // lane bases of the transposed reads from the one of (ct 0, half 0):
        // column block ct flips address bit 6, half 1 flips bit 5 and adds
        // 8 rows (the 1024 rides in the read's offset)
        const lds_char* ktr[2][2];
        const uint32_t t00 = (uint32_t)(uintptr_t)lane_tile(kring[st], tb00);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                ktr[ct][hf] = (const lds_char*)(uintptr_t)(t00 ^ ((uint32_t)ct << 6) ^
                                                             ((uint32_t)hf << 5)) +
                              1024 * hf;
#pragma unroll
        for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                dqt[ct] = mfma16<DT>(btr_at(ktr[ct][0], ktr[ct][1], 2 * nt + kl), sf[kl],
                                     dqt[ct]);
    };
    auto tile = [&](int u, v16f32& sa, v16f32& sb, auto next_tag, auto edge_tag) {
        half(u, 0, sa, sb, Y(), edge_tag);
        half(u, 1, sb, sa, next_tag, edge_tag);
    };
    auto sync_issue = [&](int u) {
        if (u > 0) {
            wait_vmcnt<0>();
            __syncthreads();
        }
        if (u + 2 < n) issue(u + 2);
    };

    if (n >= 1) issue(0);
    if (n >= 2) issue(1);
    wait_vmcnt<0>();
    __syncthreads();
    int u = 0;
    if (nw > 0) {
        v16f32 sa, sb;
        {
            v4u32 f[4];
            rows4(kring[0], 0, f);
            prod4(f, qf, sa);  // S^T of the first half of tile 0
        }
        // Only the wave's last tile can need masks (bwd_q_edge in
        // fused_layout.h; the host check walks every tile, wave and
        // length), so the loop before it runs without masks and the last
        // tile always takes the masked form.
        for (; u + 1 < nw; ++u) {
            sync_issue(u);
            tile(u, sa, sb, Y(), N());
        }
        sync_issue(u);
        tile(u, sa, sb, N(), Y());
        ++u;
    }
    for (; u < n; ++u) sync_issue(u);  // tiles past the wave's last query
    if (my_q < T) store_rows<DT>(dq + base + (int64_t)my_q * kHeadDim, dqt, scale, hh);
}

// ---------------------------------------------------------------------------
// Launcher and kernel table.
// ---------------------------------------------------------------------------
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* ws, int BH, int T, int causal, float c, float scale,
                      bool negate, int dt, hipStream_t stream) {
    const uint32_t sign = negate ? 0x80008000u : 0u;
    const int64_t rows = (int64_t)BH * T;
    float* ndelta = ws;
    float* lse2 = ws + bwd_ws_stride(rows);
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
                           dim3(256), 0, stream, o16, d16, lse, ndelta, lse2, rows);
        auto kv = causal ? bwd_kv16<ATTN_DT_BF16, true> : bwd_kv16<ATTN_DT_BF16, false>;
        hipLaunchKernelGGL(kv, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse2, ndelta, (uint16_t*)dk, (uint16_t*)dv, T, nkb, c, scale,
                           sign);
        auto qk = causal ? bwd_q16<ATTN_DT_BF16, true> : bwd_q16<ATTN_DT_BF16, false>;
        hipLaunchKernelGGL(qk, dim3((unsigned)(nq * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse2, ndelta, (uint16_t*)dq, T, nq, c, scale, sign);
    } else {
        hipLaunchKernelGGL(bwd_delta16<ATTN_DT_F16>, dim3((unsigned)((rows + 31) / 32)),
                           dim3(256), 0, stream, o16, d16, lse, ndelta, lse2, rows);
        auto kv = causal ? bwd_kv16<ATTN_DT_F16, true> : bwd_kv16<ATTN_DT_F16, false>;
        hipLaunchKernelGGL(kv, dim3((unsigned)(nkb * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse2, ndelta, (uint16_t*)dk, (uint16_t*)dv, T, nkb, c, scale,
                           sign);
        auto qk = causal ? bwd_q16<ATTN_DT_F16, true> : bwd_q16<ATTN_DT_F16, false>;
        hipLaunchKernelGGL(qk, dim3((unsigned)(nq * BH)), block, 0, stream, q16, k16, v16,
                           d16, lse2, ndelta, (uint16_t*)dq, T, nq, c, scale, sign);
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
