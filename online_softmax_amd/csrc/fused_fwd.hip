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
//  - 16-bit K and V tiles go straight from HBM to LDS by direct buffer loads
//    (buffer_load_dwordx4 ... lds) into XOR-swizzled rings of their own, K
//    four tiles deep and issued three ahead, V four deep and two ahead;
//    one barrier per tile. V^T fragments come from transposing LDS reads
//    (ds_read_b64_tr_b16), so V is stored as it arrives.
//  - S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}
//    (fp32 inputs: v_mfma_f32_32x32x2_f32 from VGPR-staged, padded LDS
//    tiles), fp32 accumulation; the 16-bit main loop is a three-stage
//    software pipeline with a lazily moved softmax reference.
//  - fp32 on grids too small to fill the CUs (one head of a few thousand
//    tokens): eight waves share 32 query rows and split the key tiles among
//    them, each staging its own tiles, and merge their partial results
//    through LDS at the end (fused_fwd32_split).
//  - Row max / row sum: in-lane, then one v_permlane32_swap between halves.
//  - Masks only on the diagonal and ragged tiles; tiles a whole wave cannot
//    see are skipped by that wave (it still joins every barrier).
// Index arithmetic lives in fused_layout.h (host-checkable).
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

// ---------------------------------------------------------------------------
// 16-bit inputs (bf16 or f16), fp32 accumulation.
// c = |scale| * log2(e); qsign = 0x80008000 negates Q for a negative scale.
// ---------------------------------------------------------------------------

// A lane's LDS fragment addresses within a tile: one per K step (ko, the key
// half-tile nt adds kKfragNtStride) and one per V half-tile (vo, the step ks
// and half add kVtrKsStride and kVtrHalfStride).
struct FragAddr {
    uint32_t ko[4];
    uint32_t vo[2];
};

// K fragments of one 64-key tile from a swizzled LDS K tile, and the product
// S^T = K Q^T (two independent accumulation chains, interleaved).
__device__ inline void kfrag16(const char* __restrict__ kb, v4u32 (&kf)[2][4],
                               const FragAddr& fa) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            kf[nt][ks] = *(const v4u32*)(kb + fa.ko[ks] + kKfragNtStride * nt);
}
template <int DT>
__device__ inline void qk16_mfma(const v4u32 (&kf)[2][4], const v4u32 (&qf)[4],
                                 v16f32 (&s)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s[nt] = mfma16<DT>(kf[nt][ks], qf[ks], s[nt]);
}
template <int DT>
__device__ inline void qk16(const char* __restrict__ kb, const v4u32 (&qf)[4],
                            v16f32 (&s)[2], const FragAddr& fa) {
    v4u32 kf[2][4];
    kfrag16(kb, kf, fa);
    qk16_mfma<DT>(kf, qf, s);
}

// V^T fragments of one 64-key tile, by transposed LDS reads.
__device__ inline void vfrag16(const char* __restrict__ vb, v4u32 (&vf)[2][4],
                               const FragAddr& fa) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        // one address per half-tile; the compiler must not split it into
        // per-read invariant sums, so the constant steps stay in the
        // instructions' offset field
        uint32_t addr = (uint32_t)(uintptr_t)(lds_void*)vb + fa.vo[mt];
        asm("" : "+v"(addr));
        typedef __attribute__((address_space(3))) char lds_char;
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        lds_char* pm = (lds_char*)addr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            lds_char* p = pm + kVtrKsStride * ks;
            const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
            const v4i16 b =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + kVtrHalfStride));
            const v2u32 a2 = __builtin_bit_cast(v2u32, a), b2 = __builtin_bit_cast(v2u32, b);
            vf[mt][ks] = (v4u32){a2[0], a2[1], b2[0], b2[1]};
        }
    }
}

// O^T += V^T P^T (two independent accumulation chains, interleaved).
template <int DT>
__device__ inline void pv16(const v4u32 (&vf)[2][4], const v4u32 (&pf)[4],
                            v16f32 (&oacc)[2]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            oacc[mt] = mfma16<DT>(vf[mt][ks], pf[ks], oacc[mt]);
}

// Instruction order of one pipelined iteration: the LDS fragment reads
// first, then a block of vector work long enough to cover their latency
// (48 instructions: measured 4% faster than none, 12 to 40 gain less, 64
// to 128 no more and 64 already spills a register), then each matrix
// product followed by an equal share of the rest, so the first product does
// not wait on the reads with nothing else to issue.
template <int NMFMA, int NVALU>
__device__ inline void sched_iteration() {
    __builtin_amdgcn_sched_group_barrier(0x002, 48, 0);  // VALU
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);  // VALU
    }
}

// Row maximum of an unmasked S^T tile and the lazy reference update.
__device__ inline void lazy_update(const v16f32 (&s)[2], v16f32 (&oacc)[2],
                                   RowState& st, float c) {
    float mx = s[0][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
    mx = halves_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx * c - st.mc > kLazyLog2) != 0) {
        const float m_new = fmaxf(st.m, mx);
        const float mc_new = m_new * c;
        const float corr = fast_exp2(st.mc - mc_new);
        st.m = m_new;
        st.mc = mc_new;
        st.l *= corr;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
    }
}

// Weights of a main tile against the current reference (no mask, no max):
// p = exp2(s*c - m*c) rounded into the P fragment; returns this lane's sum of
// the rounded p.
template <int DT>
__device__ inline float weights16(const v16f32 (&s)[2], v4u32 (&pf)[4], float mc,
                                  float c) {
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int nt = ks >> 1, r0 = (ks & 1) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p0 = fast_exp2(fmaf(s[nt][r0 + 2 * i], c, -mc));
            const float p1 = fast_exp2(fmaf(s[nt][r0 + 2 * i + 1], c, -mc));
            pf[ks][i] = pack2<DT>(p0, p1);
            if (i & 1)
                t1 = sum2<DT>(pf[ks][i], t1);
            else
                t0 = sum2<DT>(pf[ks][i], t0);
        }
    }
    return t0 + t1;
}

// The lazy check of a main tile, taken after its weights: a lane's 32 weights
// are each at most their sum t, so t <= 2^kLazyLog2 in every lane keeps every
// weight within the bound without a row maximum (an overflow to inf fails the
// test too). Otherwise (rare) S is recomputed from the K tile still in LDS,
// the reference moves to the row maximum, O and l (which hold the earlier
// tiles only) are rescaled and the weights recomputed.
template <int DT>
__device__ inline void lazy_check(const char* __restrict__ kb,
                                  const v4u32 (&qf)[4], v4u32 (&pf)[4], float t,
                                  v16f32 (&oacc)[2], RowState& st, float c,
                                  const FragAddr& fa) {
    if (__builtin_amdgcn_ballot_w64(!(t <= 256.0f)) != 0) {
        v16f32 s[2];
        qk16<DT>(kb, qf, s, fa);
        lazy_update(s, oacc, st, c);
        t = weights16<DT>(s, pf, st.mc, c);
    }
    st.l += t;
}

// 4 waves, 32 query rows each. Main tiles (no mask) run as a three-stage
// software pipeline: iteration j takes the weights of tile j (vector ALU)
// while the matrix cores compute S(j+1) = K(j+1) Q^T and O += V(j-1) P(j-1),
// none of which waits for this iteration's vector work; the lazy check of
// tile j closes the iteration. The (at most two) edge tiles run one at a time
// with masks. K and V tiles arrive by direct global -> LDS loads into rings
// of their own, K three tiles ahead and V two (schedule in fused_layout.h);
// K(j) stays resident through iteration j for the rare rescale.
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fused_fwd16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    constexpr int BN = kBlockN16;
    __shared__ __attribute__((aligned(1024))) char kring[kRingK][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char vring[kRingV][kTileBytes16];

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
    const int n_main = main_tiles(qt, T, BN, CAUSAL);

    v4u32 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T)
            x = *(const v4u32*)(qh + (int64_t)my_q * kHeadDim + q_col16(hh, ks));
        qf[ks] = x ^ qsign;
    }
    wait_vmcnt<0>();  // Q is in registers before the ring loads start

    // Direct loads (2 wave instructions, 16 bytes per lane, per K or V tile)
    // from the slice's buffer: the lane's fixed offset within a tile plus the
    // tile's offset as a scalar. The tile holding key T-1, when ragged, takes
    // per-lane offsets instead whose rows past T fetch row T-1 (a finite value
    // whose weight the edge mask sets to 0); the buffer's size (the slice)
    // bounds every access in any case.
    const uint32_t slice_bytes = (uint32_t)T * (kHeadDim * 2);
    const v4u32_rsrc krs = buffer_rsrc(kh, slice_bytes);
    const v4u32_rsrc vrs = buffer_rsrc(vh, slice_bytes);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform copy
    uint32_t kvoff[2], vvoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        kvoff[i] = (uint32_t)dl_global_byte(wave, i, lane, false);
        vvoff[i] = (uint32_t)dl_global_byte(wave, i, lane, true);
    }
    auto load_tile = [&](v4u32_rsrc rs, uint32_t off, const uint32_t(&voff)[2],
                         int tile) {
        const int k0 = __builtin_amdgcn_readfirstlane(tile) * BN;  // uniform
        if (k0 + BN <= T) {
            const uint32_t soff = (uint32_t)k0 * (kHeadDim * 2);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                dma16(rs, voff[i], soff, off + 1024 * (2 * wave_u + i));
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = min(k0 + (int)(voff[i] >> 7), T - 1);
                dma16(rs, (uint32_t)r * (kHeadDim * 2) + (voff[i] & 127), 0u,
                      off + 1024 * (2 * wave_u + i));
            }
        }
    };
    auto issue_batch = [&](int u) {
        const int tk = batch_k(u, n_tiles), tv = batch_v(u, n_tiles);
        if (tk >= 0)
            load_tile(krs, (uint32_t)(uintptr_t)(lds_void*)kring[tk % kRingK], kvoff, tk);
        if (tv >= 0)
            load_tile(vrs, (uint32_t)(uintptr_t)(lds_void*)vring[tv % kRingV], vvoff, tv);
    };
    FragAddr fa;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) fa.ko[ks] = (uint32_t)kfrag_byte(ql, hh, 0, ks);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) fa.vo[mt] = (uint32_t)vtr_byte(lane, mt, 0, 0);

    v16f32 oacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    // reference max starts finite (-FLT_MAX): no inf - inf, and scale 0 works
    RowState st = {-FLT_MAX, -FLT_MAX * c, 0.f};

    for (int u = -3; u < 0; ++u) issue_batch(u);

    // Main iteration j: S(j) is in scur (reference set for tile 0 by its row
    // maximum), P(j-1) in pprev; produces P(j) in pcur and S(j+1) in snext.
    auto main_iter = [&](int j, v16f32(&scur)[2], v16f32(&snext)[2],
                         v4u32(&pcur)[4], const v4u32(&pprev)[4], auto next_tag,
                         auto prev_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool PREV = decltype(prev_tag)::value;
        wait_loads(batch_size(j - 1, n_tiles));
        __syncthreads();
        issue_batch(j);
        v4u32 vf[2][4], kf[2][4];
        if (PREV) vfrag16(vring[(j + kRingV - 1) % kRingV], vf, fa);  // V(j-1)
        if (NEXT) kfrag16(kring[(j + 1) % kRingK], kf, fa);  // K(j+1)
        __builtin_amdgcn_sched_barrier(0);  // the reads go first
        const float t = weights16<DT>(scur, pcur, st.mc, c);
        if (PREV) pv16<DT>(vf, pprev, oacc);
        if (NEXT) qk16_mfma<DT>(kf, qf, snext);
        constexpr int NM = 8 * NEXT + 8 * PREV;
        if (NM > 0) sched_iteration<NM, 96 / (NM > 0 ? NM : 1)>();
        lazy_check<DT>(kring[j % kRingK], qf, pcur, t, oacc, st, c, fa);
    };

    bool synced = false;  // every issued load landed, all waves past a barrier
    if (n_main > 0) {
        using Y = std::integral_constant<bool, true>;
        using N = std::integral_constant<bool, false>;
        v16f32 sa[2], sb[2];
        v4u32 pa[4], pb[4];
        wait_loads(batch_size(-2, n_tiles) + batch_size(-1, n_tiles));
        __syncthreads();
        qk16<DT>(kring[0], qf, sa, fa);
        lazy_update(sa, oacc, st, c);
        // j = 0 has no product yet; then pairs so S and P ping-pong a/b
        if (n_main == 1) {
            main_iter(0, sa, sb, pa, pb, N(), N());
        } else {
            main_iter(0, sa, sb, pa, pb, Y(), N());
            int j = 1;
            for (; j + 2 < n_main; j += 2) {
                main_iter(j, sb, sa, pb, pa, Y(), Y());
                main_iter(j + 1, sa, sb, pa, pb, Y(), Y());
            }
            if (j + 1 < n_main) {
                main_iter(j, sb, sa, pb, pa, Y(), Y());
                main_iter(j + 1, sa, sb, pa, pb, N(), Y());
            } else {
                main_iter(j, sb, sa, pb, pa, N(), Y());
            }
        }
        // the last main tile's product: its P is in pa when n_main is odd
        wait_vmcnt<0>();
        __syncthreads();
        synced = true;
        v4u32 vf[2][4];
        vfrag16(vring[(n_main - 1) % kRingV], vf, fa);
        if (n_main & 1)
            pv16<DT>(vf, pa, oacc);
        else
            pv16<DT>(vf, pb, oacc);
    }
    // edge tiles (diagonal or ragged; at most two), one at a time; their K and
    // V tiles were issued by earlier batches
    for (int t = n_main; t < n_tiles; ++t) {
        if (!synced) {
            wait_vmcnt<0>();
            __syncthreads();
        }
        synced = false;
        if (!CAUSAL || t * BN <= wq0 + 31) {  // a wave skips tiles it cannot see
            v16f32 s[2];
            v4u32 vf[2][4], pf[4];
            qk16<DT>(kring[t % kRingK], qf, s, fa);
            vfrag16(vring[t % kRingV], vf, fa);
            softmax_tile<DT, CAUSAL, true, 2>(s, pf, oacc, st, c, t * BN, T, my_q, hh);
            pv16<DT>(vf, pf, oacc);
        }
    }

    const float lt = halves_sum(st.l);
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
            lse[(int64_t)bh * T + my_q] = (st.mc + log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// 8 waves, 32 query rows each (256 per workgroup), sharing every K and V
// tile: each wave fetches one eighth of a tile (one 1 KiB direct load per
// ring), so a tile's loads and its LDS writes serve twice the rows of the
// 4-wave kernel. The loop is plain (S, weights, P.V of one tile at a time,
// the lazy reference of softmax_tile), which keeps a wave within 128 VGPRs:
// two workgroups then give every SIMD four waves, and the SIMD interleaves
// one wave's matrix instructions with another's vector work instead of the
// kernel pipelining them inside one wave. Rings: K and V four tiles deep,
// tile t + 3 issued after the barrier of iteration t into the stage tile
// t - 1 used. Each wave computes only its own tiles (w8_seen) and masks only
// its own diagonal and the ragged tile (w8_main); it joins every barrier.
//
// SPLIT = kSplit8 is the key-split form for small grids: waves w and
// w + 4 own the same 32 rows (128 per workgroup), and in iteration i the
// two groups compute tiles 2i and 2i + 1, both loaded by all eight waves
// (the pair for iteration i + 1 is issued after iteration i's barrier into
// the stages of the pair before). At the end the second group hands its
// O, reference and denominator to the first through LDS, which merges
// them by the same rescale as any reference move: the reference becomes
// the larger of the two and each side is scaled by exp2(its - new).
// ---------------------------------------------------------------------------
template <int DT, bool CAUSAL, int SPLIT>
__global__ __launch_bounds__(kThreads8, 4) void fused_fwd16w8(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    static_assert(SPLIT == 1 || SPLIT == kSplit8, "one or two key groups");
    constexpr int BN = kBlockN16;
    constexpr int RW = kWaves8 / SPLIT;  // waves per key group, one per 32 rows
    constexpr int BM = 32 * RW;          // query rows per workgroup
    __shared__ __attribute__((aligned(1024))) char kring[kRing8][kTileBytes16];
    __shared__ __attribute__((aligned(1024))) char vring[kRing8][kTileBytes16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform copy
    const int rw = SPLIT == 1 ? wave_u : wave_u % RW;  // which 32 rows
    const int grp = SPLIT == 1 ? 0 : wave_u / RW;      // key group: tiles t % SPLIT == grp

    int bh, qt;
    tile_of8(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const int wq0 = qt * BM + 32 * rw;  // first query row of this wave
    const int my_q = wq0 + ql;          // this lane's query row
    const int n_tiles = key_tiles(qt, T, BN, CAUSAL, BM);
    const int n_seen = w8_seen(qt, rw, T, CAUSAL, BM);

    // Q rows first: their loads are older than every ring load, so the
    // first tile's wait covers them too
    v4u32 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T)
            x = *(const v4u32*)(q + base + (int64_t)my_q * kHeadDim + q_col16(hh, ks));
        qf[ks] = x ^ qsign;
    }

    // wave w's share of a tile: the 4-wave schedule's instruction w (rows
    // 8w .. 8w + 7); the ragged last tile clamps rows past T to row T - 1
    // (their weights are masked to 0), and the slice's buffer bounds every
    // access in any case
    const uint32_t slice_bytes = (uint32_t)T * (kHeadDim * 2);
    const v4u32_rsrc krs = buffer_rsrc(k + base, slice_bytes);
    const v4u32_rsrc vrs = buffer_rsrc(v + base, slice_bytes);
    const uint32_t kvoff = (uint32_t)dl_global_byte(wave >> 1, wave & 1, lane, false);
    const uint32_t vvoff = (uint32_t)dl_global_byte(wave >> 1, wave & 1, lane, true);
    auto load_tile = [&](v4u32_rsrc rs, const char* stage, uint32_t voff, int tile) {
        const uint32_t off = (uint32_t)(uintptr_t)(lds_void*)stage + 1024 * wave_u;
        const int k0 = tile * BN;
        if (k0 + BN <= T) {
            dma16(rs, voff, (uint32_t)k0 * (kHeadDim * 2), off);
        } else {
            const int r = min(k0 + (int)(voff >> 7), T - 1);
            dma16(rs, (uint32_t)r * (kHeadDim * 2) + (voff & 127), 0u, off);
        }
    };
    auto issue = [&](int t) {
        load_tile(krs, kring[t % kRing8], kvoff, t);
        load_tile(vrs, vring[t % kRing8], vvoff, t);
    };
    for (int t = 0; t < (SPLIT == 1 ? kAhead8 : SPLIT) && t < n_tiles; ++t) issue(t);

    // Fragment addresses from one lane base per tile each: the swizzles only
    // permute 16-byte chunks within a row and the stages are 8 KiB aligned,
    // so K step ks is base XOR (ks << 5) (the second key half adds 4096) and
    // V output block mt is base XOR (mt << 6) (steps and halves add
    // constants), checked on the host for every lane and stage.
    const uint32_t ko0 = (uint32_t)kfrag_byte(ql, hh, 0, 0);
    const uint32_t vo0 = (uint32_t)vtr_byte(lane, 0, 0, 0);

    v16f32 oacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    // reference max starts finite (-FLT_MAX): no inf - inf, and scale 0 works
    RowState st = {-FLT_MAX, -FLT_MAX * c, 0.f};

    // One tile. The fragment reads are written in groups of four (16
    // registers) and the compiler orders them within the 128-VGPR budget;
    // the LDS latency a wave waits out is covered by the SIMD's other waves.
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) v4u32 lds_v4u32;
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    auto step = [&](int t, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        uint32_t ka = (uint32_t)(uintptr_t)(lds_void*)kring[t % kRing8] + ko0;
        uint32_t va = (uint32_t)(uintptr_t)(lds_void*)vring[t % kRing8] + vo0;
        asm("" : "+v"(ka), "+v"(va));  // one address each; constants ride in offsets
        v16f32 s[2];
        v4u32 f[4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                f[ks] = *(const lds_v4u32*)((const lds_char*)(uintptr_t)(ka ^ ((uint32_t)ks << 5)) +
                                            kKfragNtStride * nt);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s[nt] = mfma16<DT>(f[ks], qf[ks], s[nt]);
        }
        v4u32 pf[4];
        softmax_tile<DT, CAUSAL, EDGE, 2>(s, pf, oacc, st, c, t * BN, T, my_q, hh);
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ks = 2 * kp + (j >> 1), mt = j & 1;
                const lds_char* p =
                    (const lds_char*)(uintptr_t)(va ^ ((uint32_t)mt << 6)) + kVtrKsStride * ks;
                const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
                const v4i16 b =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + kVtrHalfStride));
                const v2u32 a2 = __builtin_bit_cast(v2u32, a), b2 = __builtin_bit_cast(v2u32, b);
                f[j] = (v4u32){a2[0], a2[1], b2[0], b2[1]};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ks = 2 * kp + (j >> 1), mt = j & 1;
                oacc[mt] = mfma16<DT>(f[j], pf[ks], oacc[mt]);
            }
        }
    };
    auto sync_issue = [&](int t) {
        if (SPLIT == 1) {
            // this wave's loads of tile t (and the Q rows) have landed; those
            // of the (up to two) later tiles already issued may still be in
            // flight
            const int ahead = min(kAhead8 - 1, n_tiles - 1 - t);
            if (ahead >= 2)
                wait_vmcnt<4>();
            else if (ahead == 1)
                wait_vmcnt<2>();
            else
                wait_vmcnt<0>();
            __syncthreads();  // everyone's share landed; tile t - 1's stages are free
            if (t + kAhead8 < n_tiles) issue(t + kAhead8);
        } else {
            // t is the iteration: its pair of tiles (and the Q rows) landed
            wait_vmcnt<0>();
            __syncthreads();  // the previous pair's stages are free
#pragma unroll
            for (int j = 0; j < SPLIT; ++j)
                if (SPLIT * (t + 1) + j < n_tiles) issue(SPLIT * (t + 1) + j);
        }
    };
    // Tiles every wave computes unmasked (those before the first wave's
    // first masked one), then the last few (at most four), where each wave
    // takes the masked step on every tile it sees: on a tile that needs no
    // mask it masks nothing and takes the same decisions, so the results
    // are the same bits, and one step form keeps the tail within the
    // register budget.
    // (key split: iteration i, tile SPLIT * i + grp; the unmasked loop runs
    // while both tiles of the pair are unmasked for every wave)
    const int n_all_main = w8_main(qt, 0, T, CAUSAL, BM);
    const int n_iter = (n_tiles + SPLIT - 1) / SPLIT;
    int i = 0;
    for (; i < n_all_main / SPLIT; ++i) {
        sync_issue(i);
        const int t = SPLIT * i + grp;
        if (t < n_seen) step(t, std::integral_constant<bool, false>());  // rows < T
    }
    for (; i < n_iter; ++i) {
        sync_issue(i);
        const int t = SPLIT * i + grp;
        if (t < n_seen) step(t, std::integral_constant<bool, true>());
    }
    if (SPLIT > 1) {
        // group 1 hands O, mc and l (lane by lane: the partner lane holds the
        // same row and dims) to group 0 through the rings, now free
        __syncthreads();
        float* xo = (float*)&kring[0][0];  // [RW][32][64]: 32 KiB
        float* xs = (float*)&vring[0][0];  // [RW][2][64]
        if (grp == 1) {
#pragma unroll
            for (int r = 0; r < 32; ++r) xo[(rw * 32 + r) * 64 + lane] = oacc[r >> 4][r & 15];
            xs[(rw * 2) * 64 + lane] = st.mc;
            xs[(rw * 2 + 1) * 64 + lane] = st.l;
        }
        __syncthreads();
        if (grp != 0) return;
        const float mc1 = xs[(rw * 2) * 64 + lane], l1 = xs[(rw * 2 + 1) * 64 + lane];
        const float mcn = fmaxf(st.mc, mc1);
        const float a0 = fast_exp2(st.mc - mcn), a1 = fast_exp2(mc1 - mcn);
#pragma unroll
        for (int r = 0; r < 32; ++r)
            oacc[r >> 4][r & 15] = oacc[r >> 4][r & 15] * a0 + xo[(rw * 32 + r) * 64 + lane] * a1;
        st.l = st.l * a0 + l1 * a1;
        st.mc = mcn;
    }

    // the output row from an opaque copy of the thread index, so its address
    // is not computed before the loop and carried through it
    int tid_late = tid;
    asm("" : "+v"(tid_late));
    const int row =
        qt * BM + 32 * (SPLIT == 1 ? tid_late >> 6 : (tid_late >> 6) % RW) + (tid_late & 31);
    const float lt = halves_sum(st.l);
    const float inv = 1.0f / lt;
    if (row < T) {
        uint16_t* orow = o + base + (int64_t)row * kHeadDim;
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
        if (lse != nullptr && (tid_late & 32) == 0)
            lse[(int64_t)bh * T + row] = (st.mc + log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same schedule on v_mfma_f32_32x32x2_f32, 32-key tiles,
// fp32 weights (no lazy path: this kernel is bound by the fp32 matrix rate).
// qsign = 0x80000000 negates Q for a negative scale.
// ---------------------------------------------------------------------------
template <bool CAUSAL, bool EDGE>
__device__ inline void tile32(const float* __restrict__ skb,
                              const float* __restrict__ svb,
                              const v4f32 (&qf)[8], v16f32 (&oacc)[2],
                              RowState& st, float c, int k0, int T, int my_q,
                              int ql, int hh) {
    v16f32 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const v4f32 kf = *(const v4f32*)&skb[kfrag32(ql, hh, g)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i], qf[g][i], s, 0, 0,
                                                      0);
    }
    if (EDGE) {
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
    const float m_new = fmaxf(st.m, mx);
    const float mc_new = m_new * c;
    const float corr = fast_exp2(st.mc - mc_new);
    st.m = m_new;
    st.mc = mc_new;
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(s[r], c, -mc_new));
        if (EDGE && s[r] == -INFINITY) p = 0.f;
        s[r] = p;
        if (r & 1)
            t1 += p;
        else
            t0 += p;
    }
    st.l = st.l * corr + (t0 + t1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
    // O^T += V^T P^T: step 4g + i pairs key 8g + 4h + i of each half with
    // accumulator register 4g + i of the score tile.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v4f32 vf = *(const v4f32*)&svb[vfrag32(ql, hh, mt, g)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    vf[i], s[4 * g + i], oacc[mt], 0, 0, 0);
        }
}

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
    const int n_main = main_tiles(qt, T, BN, CAUSAL);

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
    RowState st = {-FLT_MAX, -FLT_MAX * c, 0.f};

    auto step = [&](int kt, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) gload(kt + 1);
        const int k0 = kt * BN;
        if (!EDGE || !CAUSAL || k0 <= wq0 + 31)
            tile32<CAUSAL, EDGE>(sk[buf], sv[buf], qf, oacc, st, c, k0, T, my_q,
                                 ql, hh);
        if (more) lstore(buf ^ 1);
        __syncthreads();
    };
    int kt = 0;
    for (; kt < n_main; ++kt) step(kt, std::integral_constant<bool, false>());
    for (; kt < n_tiles; ++kt) step(kt, std::integral_constant<bool, true>());

    const float lt = halves_sum(st.l);
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
            lse[(int64_t)bh * T + my_q] = (st.mc + log2f(lt)) * kLn2;
    }
}

// fp32 inputs, small grids: kSplitWaves waves share 32 query rows and split
// the key tiles among them (wave w: tiles w, w + kSplitWaves, ...), each with
// its own LDS tile, no barrier until the end; then the partial results merge
// by the online-softmax combination O = sum_w 2^(m_w c - m c) O_w over
// sum_w 2^(m_w c - m c) l_w, m the largest m_w.
template <bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads, 1) void fused_fwd32_split(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, int T, int nq, float c, uint32_t qsign) {
    constexpr int BN = kBlockN32;
    __shared__ __attribute__((aligned(16))) float lds[kSplitWaves][kSplitTileFloats];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    tile_of(blockIdx.x, gridDim.x, nq, CAUSAL, &bh, &qt);
    const int64_t base = (int64_t)bh * T * kHeadDim;
    const float* kh = k + base;
    const float* vh = v + base;
    const int q0 = qt * kSplitRows;
    const int my_q = q0 + ql;
    const int n_tiles = key_tiles(qt, T, BN, CAUSAL, kSplitRows);
    const int n_main = main_tiles(qt, T, BN, CAUSAL, kSplitRows);

    v4f32 qf[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < T)
            x = *(const v4u32*)(q + base + (int64_t)my_q * kHeadDim + q_col32(hh, g));
        qf[g] = __builtin_bit_cast(v4f32, x ^ qsign);
    }

    // The wave stages its tiles alone: lane l does the work of threads
    // l + 64 j (j < 4) of the 256-thread staging pattern.
    float* const sk = lds[wave];
    float* const sv = lds[wave] + kKTile32;
    v4f32 kr[8], vr[8];
    auto gload = [&](int kt) {
        const int k0 = kt * BN;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = lane + 64 * j;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int row, col;
                k_stage32(t, i, &row, &col);
                v4f32 x = {0.f, 0.f, 0.f, 0.f};
                if (k0 + row < T) x = *(const v4f32*)(kh + (int64_t)(k0 + row) * kHeadDim + col);
                kr[2 * j + i] = x;
            }
            int key0, dim0;
            v_stage32(t, &key0, &dim0);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                v4f32 x = {0.f, 0.f, 0.f, 0.f};
                if (k0 + key0 + e < T)
                    x = *(const v4f32*)(vh + (int64_t)(k0 + key0 + e) * kHeadDim + dim0);
                vr[2 * j + e] = x;
            }
        }
    };
    // LDS reads and writes of one wave complete in order, so the next tile
    // may overwrite the one the wave has just read without a barrier.
    auto lstore = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = lane + 64 * j;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int row, col;
                k_stage32(t, i, &row, &col);
                *(v4f32*)&sk[k_lds32(row, col)] = kr[2 * j + i];
            }
            int key0, dim0;
            v_stage32(t, &key0, &dim0);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float2 w;
                w.x = vr[2 * j][d];
                w.y = vr[2 * j + 1][d];
                *(float2*)&sv[v_lds32(dim0 + d, key0)] = w;
            }
        }
    };

    v16f32 oacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
    RowState st = {-FLT_MAX, -FLT_MAX * c, 0.f};

    auto step = [&](int kt, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const bool more = kt + kSplitWaves < n_tiles;
        if (more) gload(kt + kSplitWaves);
        tile32<CAUSAL, EDGE>(sk, sv, qf, oacc, st, c, kt * BN, T, my_q, ql, hh);
        if (more) lstore();
    };
    int kt = wave;
    if (kt < n_tiles) {
        gload(kt);
        lstore();
    }
    for (; kt < n_main; kt += kSplitWaves) step(kt, std::integral_constant<bool, false>());
    for (; kt < n_tiles; kt += kSplitWaves) step(kt, std::integral_constant<bool, true>());

    // Merge: each wave's partial O (rows = queries, stride kMergeStride32),
    // reference m*c and denominator into LDS, then thread t finishes dims
    // 4 (t % 16) .. + 3 of row t / 16.
    __syncthreads();
    float* const obuf = &lds[0][0];
    float* const mlbuf = obuf + kSplitWaves * kSplitRows * kMergeStride32;
    {
        float* ow = obuf + wave * kSplitRows * kMergeStride32 + ql * kMergeStride32;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) ow[32 * mt + acc_row(r, hh)] = oacc[mt][r];
        const float lt = halves_sum(st.l);
        if (hh == 0) {
            mlbuf[2 * (wave * kSplitRows + ql)] = st.mc;
            mlbuf[2 * (wave * kSplitRows + ql) + 1] = lt;
        }
    }
    __syncthreads();
    const int row = tid >> 4, d0 = 4 * (tid & 15);
    float mcmax = mlbuf[2 * row];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) mcmax = fmaxf(mcmax, mlbuf[2 * (w * kSplitRows + row)]);
    float den = 0.f;
    v4f32 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
        const float a = fast_exp2(mlbuf[2 * (w * kSplitRows + row)] - mcmax);
        den = fmaf(a, mlbuf[2 * (w * kSplitRows + row) + 1], den);
        const float* ow = obuf + (w * kSplitRows + row) * kMergeStride32 + d0;
#pragma unroll
        for (int i = 0; i < 4; ++i) num[i] = fmaf(a, ow[i], num[i]);
    }
    if (q0 + row < T) {
        const float inv = 1.0f / den;
        v4f32 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = num[i] * inv;
        *(v4f32*)(o + base + (int64_t)(q0 + row) * kHeadDim + d0) = w;
        if (lse != nullptr && (tid & 15) == 0)
            lse[(int64_t)bh * T + q0 + row] = (mcmax + log2f(den)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Launchers and the kernel table.
// ---------------------------------------------------------------------------
hipError_t launch_fused(const void* q, const void* k, const void* v, void* o,
                        float* lse, int BH, int T, int causal, float c,
                        bool negate_q, int dt, hipStream_t stream) {
    if (dt == ATTN_DT_F32) {
        const uint32_t sign = negate_q ? 0x80000000u : 0u;
        if (fwd32_split(BH, T)) {
            const int nq = (T + kSplitRows - 1) / kSplitRows;
            auto fn = causal ? fused_fwd32_split<true> : fused_fwd32_split<false>;
            hipLaunchKernelGGL(fn, dim3((unsigned)(nq * BH)), dim3(kSplitThreads), 0, stream,
                               (const float*)q, (const float*)k, (const float*)v, (float*)o,
                               lse, T, nq, c, sign);
        } else {
            const int nq = (T + kBlockM - 1) / kBlockM;
            auto fn = causal ? fused_fwd32<true> : fused_fwd32<false>;
            hipLaunchKernelGGL(fn, dim3((unsigned)(nq * BH)), dim3(kThreads), 0, stream,
                               (const float*)q, (const float*)k, (const float*)v, (float*)o,
                               lse, T, nq, c, sign);
        }
    } else if (fwd16_eight_waves(BH, T, causal != 0) || fwd16_key_split(BH, T, causal != 0)) {
        const bool split = !fwd16_eight_waves(BH, T, causal != 0);
        const int bm = split ? kBlockM8s : kBlockM8;
        const int nq = (T + bm - 1) / bm;
        const dim3 grid((unsigned)(nq * BH));
        const dim3 block(kThreads8);
        const uint32_t sign = negate_q ? 0x80008000u : 0u;
        const int index = (split ? 4 : 0) + (dt == ATTN_DT_F16 ? 2 : 0) + (causal ? 0 : 1);
        auto fn = (void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                            int, int, float, uint32_t))fused_w8_kernel_ptr(index);
        hipLaunchKernelGGL(fn, grid, block, 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                           (const uint16_t*)v, (uint16_t*)o, lse, T, nq, c, sign);
    } else {
        const int nq = (T + kBlockM - 1) / kBlockM;
        const dim3 grid((unsigned)(nq * BH));
        const dim3 block(kThreads);
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
        case 6: return (const void*)fused_fwd32_split<true>;
        case 7: return (const void*)fused_fwd32_split<false>;
        default: return nullptr;
    }
}

// Table order: the eight-wave kernel, then its key-split form; bf16 then
// f16; causal then not.
const void* fused_w8_kernel_ptr(int index) {
    switch (index) {
        case 0: return (const void*)fused_fwd16w8<ATTN_DT_BF16, true, 1>;
        case 1: return (const void*)fused_fwd16w8<ATTN_DT_BF16, false, 1>;
        case 2: return (const void*)fused_fwd16w8<ATTN_DT_F16, true, 1>;
        case 3: return (const void*)fused_fwd16w8<ATTN_DT_F16, false, 1>;
        case 4: return (const void*)fused_fwd16w8<ATTN_DT_BF16, true, kSplit8>;
        case 5: return (const void*)fused_fwd16w8<ATTN_DT_BF16, false, kSplit8>;
        case 6: return (const void*)fused_fwd16w8<ATTN_DT_F16, true, kSplit8>;
        case 7: return (const void*)fused_fwd16w8<ATTN_DT_F16, false, kSplit8>;
        default: return nullptr;
    }
}

}  // namespace attn
