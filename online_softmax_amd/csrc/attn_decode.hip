// Attention of a few new queries against a key/value cache (decode) for
// gfx950: Tq queries, Tk cached keys and values per (batch, head) slice,
// query i standing at position Tk - Tq + i, so the causal mask is aligned to
// the bottom-right of the Tq x Tk table. "Flash attention in PyTorch, then
// in Triton" names this case (new tokens against all the keys, section
// "Backwards, and training with it") as one its kernel does not handle.
//
// With few queries there is too little work per slice to fill the GPU along
// the queries, so the keys are split: decode_split16 gives every workgroup
// one query tile (32 rows) and one range of keys, and writes a partial
// result normalised by its own denominator together with its log-sum-exp;
// decode_combine16 then merges the partials of a row with the same identity
// the online softmax uses between key tiles: with lse = log sum_s exp(lse_s),
// O = sum_s exp(lse_s - lse) O_s.
//
// Inside a workgroup each of the 4 waves takes every fourth 32-key tile of
// the range, streamed by direct buffer loads into an LDS ring of its own (no
// barrier until the end), and keeps its own online-softmax state; S^T = K Q^T
// and O^T += V^T P^T run on v_mfma_f32_32x32x16 exactly as in the forward
// kernel (fused_fwd.hip), half-height K/V tiles. The four states are merged
// through LDS at the end. The path moves the K/V cache once: it is bound by
// HBM bandwidth.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fused_layout.h"
#include "gfx950.h"
#include "kernels.h"

namespace attn {

constexpr float kDecLn2 = 0.693147180559945309417f;

// One 32-key tile of K or V (head dimension D) into `off` (D / 16 wave
// instructions): rows from row0, rows at or past `rows_end` fetch row
// rows_end - 1 (their weight is masked to 0).
template <int D>
__device__ inline void dec_load(v4u32_rsrc rs, const uint32_t (&voff)[dec_instr<D>()],
                                int row0, int rows_end, uint32_t off) {
    constexpr uint32_t kRow = HeadDim<D>::kRowBytes;
    if (row0 + kDecTile <= rows_end) {
        const uint32_t soff = (uint32_t)row0 * kRow;
#pragma unroll
        for (int i = 0; i < dec_instr<D>(); ++i) dma16(rs, voff[i], soff, off + 1024 * i);
    } else {
#pragma unroll
        for (int i = 0; i < dec_instr<D>(); ++i) {
            const int r = min(row0 + (int)(voff[i] / kRow), rows_end - 1);
            dma16(rs, (uint32_t)r * kRow + voff[i] % kRow, 0u, off + 1024 * i);
        }
    }
}

// Partial results of one split: o_part [rows, nsplit, D] float32 (normalised
// by the split's own denominator), lse_part [rows, nsplit] (natural log; -inf
// where the split holds no visible key of the row). rows = BH * Tq.
// At D = 128 the ring (128 KiB) leaves room for one workgroup per CU, which
// is all the split plan launches.
//
// MERGED (the no-allocation entry point): the partials live in the library's
// own scratch, and the last workgroup of a query tile to finish merges them
// into o and lse itself (one launch, no combine kernel). Each tile has a
// counter that starts at 0; a workgroup publishes its partial (release at
// device scope), then adds 1 to the counter; the one that reads nsplit - 1
// acquires, merges, and sets the counter back to 0 for the next call. With
// one split the workgroup writes o and lse directly.
template <int DT, bool CAUSAL, int D, bool MERGED = false>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void decode_split16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Tq, int Tk, int nqt, int nsplit, int chunk, float c, uint32_t qsign,
    uint16_t* __restrict__ o, float* __restrict__ lse, uint32_t* __restrict__ counters) {
    using G = HeadDim<D>;
    // ring depth per wave (four stages were measured no faster at D = 64)
    constexpr int kStages = 2;
    constexpr int NI = dec_instr<D>();     // direct loads per K or V tile
    constexpr int NK = G::kSteps, NO = G::kOTiles;
    constexpr int kTile = dec_tile_bytes<D>();
    __shared__ __attribute__((aligned(1024))) char ring[kWaves][kStages][2][kTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;
    const int hh = lane >> 5;

    // block -> (slice, query tile, split); splits of one slice are adjacent
    const int per_slice = nqt * nsplit;
    const int bh = blockIdx.x / per_slice;
    const int rem = blockIdx.x - bh * per_slice;
    const int qt = rem / nsplit;
    const int split = rem - qt * nsplit;
    const int my_q = qt * kDecTile + ql;  // this lane's query (0 .. Tq-1 valid)

    // keys this split covers, cut at the last key any query of the tile sees
    const int last_q = min(qt * kDecTile + kDecTile - 1, Tq - 1);
    const int kend_all = CAUSAL ? (Tk - Tq + last_q + 1) : Tk;
    const int k_begin = split * chunk;
    const int k_end = min(k_begin + chunk, kend_all);
    // this lane's first invisible key
    const int limit = min(k_end, CAUSAL ? (Tk - Tq + my_q + 1) : Tk);

    const uint32_t slice_bytes = (uint32_t)Tk * G::kRowBytes;
    const int64_t kv_base = (int64_t)bh * Tk * D;
    const v4u32_rsrc krs = buffer_rsrc(k + kv_base, slice_bytes);
    const v4u32_rsrc vrs = buffer_rsrc(v + kv_base, slice_bytes);
    uint32_t kvoff[NI], vvoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        kvoff[i] = (uint32_t)G::global_byte(i, lane, false);
        vvoff[i] = (uint32_t)G::global_byte(i, lane, true);
    }
    // this wave's tiles: k_begin + 32 * (wave + 4 t), t = 0 .. n - 1
    const int ntile_all = k_end > k_begin ? (k_end - k_begin + kDecTile - 1) / kDecTile : 0;
    const int n = ntile_all > wave ? (ntile_all - wave + kWaves - 1) / kWaves : 0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform copy
    auto issue = [&](int t) {
        const int k0 = k_begin + kDecTile * (wave_u + kWaves * t);
        const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)ring[wave_u][t % kStages][0];
        dec_load<D>(krs, kvoff, k0, k_end, base);
        dec_load<D>(vrs, vvoff, k0, k_end, base + kTile);
    };

    // lane bases of the fragment reads (the swizzles depend on the lane only)
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
    float m = -FLT_MAX, mc = -FLT_MAX * c, l = 0.f;

    // the Q rows, then the first kStages tiles: the latencies overlap, and
    // waiting for Q (older than the tiles) waits for no tile
    v4u32 qf[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        v4u32 x = {0u, 0u, 0u, 0u};
        if (my_q < Tq)
            x = *(const v4u32*)(q + ((int64_t)bh * Tq + my_q) * D + G::q_col(hh, ks));
        qf[ks] = x ^ qsign;
    }
#pragma unroll
    for (int st = 0; st < kStages; ++st)
        if (n > st) issue(st);
    for (int t = 0; t < n; ++t) {
        // tile t landed; the later tiles already issued (2 NI loads each)
        // may stay in flight
        const int ahead = min(kStages - 1, n - 1 - t);
        if (kStages > 3 && ahead >= 3)
            wait_vmcnt<(kStages > 3 ? 3 : 0) * 2 * NI>();
        else if (kStages > 2 && ahead >= 2)
            wait_vmcnt<(kStages > 2 ? 2 : 0) * 2 * NI>();
        else if (ahead >= 1)
            wait_vmcnt<2 * NI>();
        else
            wait_vmcnt<0>();
        const char* kb = ring[wave][t % kStages][0];
        const char* vb = ring[wave][t % kStages][1];
        const int k0 = k_begin + kDecTile * (wave + kWaves * t);
        // S^T = K Q^T (32 keys x 32 queries)
        v16f32 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
            s = mfma16<DT>(*(const v4u32*)(kb + ko[ks]), qf[ks], s);
        // mask, running maximum, rescale
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (k0 + acc_row(r, hh) >= limit) s[r] = -INFINITY;
            mx = fmaxf(mx, s[r]);
        }
        mx = halves_max(mx);
        const float m_new = fmaxf(m, mx);
        const float mc_new = m_new * c;
        const float corr = fast_exp2(mc - mc_new);
        m = m_new;
        mc = mc_new;
        l *= corr;
#pragma unroll
        for (int mt = 0; mt < NO; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
        // weights of the tile's 32 keys: P fragments of two 16-key steps
        v4u32 pf[2];
        float t0 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 8 * ks + 2 * i;
                float p0 = fast_exp2(fmaf(s[r], c, -mc));
                float p1 = fast_exp2(fmaf(s[r + 1], c, -mc));
                if (s[r] == -INFINITY) p0 = 0.f;
                if (s[r + 1] == -INFINITY) p1 = 0.f;
                pf[ks][i] = pack2<DT>(p0, p1);
                t0 = sum2<DT>(pf[ks][i], t0);
            }
        l += t0;
        // O^T += V^T P^T
#pragma unroll
        for (int mt = 0; mt < NO; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
                const char* p = vb + vo[mt] + 16 * G::kRowBytes * ks;
                const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
                const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(p + 8 * G::kRowBytes));
                const v2u32 a2 = __builtin_bit_cast(v2u32, a), b2 = __builtin_bit_cast(v2u32, b);
                oacc[mt] = mfma16<DT>((v4u32){a2[0], a2[1], b2[0], b2[1]}, pf[ks], oacc[mt]);
            }
        // refill the stage of tile t once its fragment reads have returned:
        // the direct loads write the LDS behind the reads' backs, so the
        // reads (issued above, consumed by matrix instructions the compiler
        // may place after this point) are waited for first
        if (t + kStages < n) {
            wait_lgkmcnt0();
            issue(t + kStages);
        }
    }

    // merge the four waves' states through LDS (the ring is free now)
    __syncthreads();
    float* so = (float*)&ring[0][0][0][0];  // [wave][32 queries][D dims]
    float* sm = so + kWaves * kDecTile * D;  // [wave][32] reference mc
    float* sl = sm + kWaves * kDecTile;      // [wave][32] denominator
    const float lt = halves_sum(l);
#pragma unroll
    for (int mt = 0; mt < NO; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            so[(wave * kDecTile + ql) * D + 32 * mt + acc_row(r, hh)] = oacc[mt][r];
    if (hh == 0) {
        sm[wave * kDecTile + ql] = mc;
        sl[wave * kDecTile + ql] = lt;
    }
    __syncthreads();
    // thread -> (query row, D / 8 dims)
    constexpr int kDims = D / 8;
    const int rq = tid >> 3, d0 = kDims * (tid & 7);
    const int qrow = qt * kDecTile + rq;
    if (qrow < Tq) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (sl[w * kDecTile + rq] > 0.f) M = fmaxf(M, sm[w * kDecTile + rq]);
        float L = 0.f, acc[kDims];
#pragma unroll
        for (int j = 0; j < kDims; ++j) acc[j] = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float lw = sl[w * kDecTile + rq];
                if (!(lw > 0.f)) continue;
                const float e = fast_exp2(sm[w * kDecTile + rq] - M);
                L += e * lw;
#pragma unroll
                for (int j = 0; j < kDims; ++j) acc[j] += e * so[(w * kDecTile + rq) * D + d0 + j];
            }
        }
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        if (MERGED && nsplit == 1) {  // the whole row: the output itself
            const int64_t row = (int64_t)bh * Tq + qrow;
#pragma unroll
            for (int j = 0; j < kDims; j += 2)
                *(uint32_t*)(o + row * D + d0 + j) = pack2<DT>(acc[j] * inv, acc[j + 1] * inv);
            if ((tid & 7) == 0 && lse != nullptr) lse[row] = (M + log2f(L)) * kDecLn2;
        } else {
            const int64_t p = ((int64_t)bh * Tq + qrow) * nsplit + split;
#pragma unroll
            for (int j = 0; j < kDims; ++j) o_part[p * D + d0 + j] = acc[j] * inv;
            if ((tid & 7) == 0) lse_part[p] = L > 0.f ? (M + log2f(L)) * kDecLn2 : -INFINITY;
        }
    }
    if constexpr (MERGED) {
        if (nsplit == 1) return;
        __shared__ int is_last;
        // Every wave's partial stores have completed before the barrier; one
        // lane then publishes them device-wide with a release on the tile's
        // counter (one cache write-back per workgroup, not one per wave).
        wait_vmcnt<0>();
        __syncthreads();
        const int tile = blockIdx.x / nsplit;  // (slice, query tile)
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            wait_vmcnt<0>();  // the write-back has completed before the count
            const uint32_t before = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            const int last = before == (uint32_t)(nsplit - 1);
            // only the last workgroup reads the other partials: it alone
            // acquires (its CU's caches drop what they held of them)
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            is_last = last;
        }
        __syncthreads();
        if (!is_last) return;
        if (qrow < Tq) {
            const int64_t row = (int64_t)bh * Tq + qrow;
            const float* lp = lse_part + row * nsplit;
            const float* op = o_part + row * nsplit * D + d0;
            float M = -INFINITY;
            for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, lp[sp]);
            float L = 0.f, acc[kDims];
#pragma unroll
            for (int j = 0; j < kDims; ++j) acc[j] = 0.f;
            for (int sp = 0; sp < nsplit; ++sp) {
                const float ls = lp[sp];
                const float e = ls == -INFINITY ? 0.f : __expf(ls - M);
                L += e;
#pragma unroll
                for (int j = 0; j < kDims; ++j) acc[j] += e * op[(int64_t)sp * D + j];
            }
            const float inv = 1.0f / L;
#pragma unroll
            for (int j = 0; j < kDims; j += 2)
                *(uint32_t*)(o + row * D + d0 + j) = pack2<DT>(acc[j] * inv, acc[j + 1] * inv);
            if ((tid & 7) == 0 && lse != nullptr) lse[row] = M + logf(L);
        }
        if (tid == 0)  // the tile's counter back to 0 for the next call
            __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Merge the nsplit partials of every row: one wave per row. Lanes take the
// splits' log-sum-exps (the maximum and the sum of the weights are wave
// reductions), then a lane per dim accumulates the weighted partials, eight
// independent loads at a time.
__device__ inline float wave_max(float x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Lane j holds dims j, j + 64, ... below D (lanes 32..63 of a D = 32 row
// repeat lanes 0..31 and store nothing).
template <int DT, int D>
__global__ __launch_bounds__(256) void decode_combine16(const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        uint16_t* __restrict__ o,
                                                        float* __restrict__ lse, int64_t rows,
                                                        int nsplit) {
    constexpr int NPL = D >= 64 ? D / 64 : 1;  // dims per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int dim = D >= 64 ? lane : (lane & (D - 1));
    const float* lp = lse_part + row * nsplit;
    const float* op = o_part + row * nsplit * D + dim;
    float M = -INFINITY;
    for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, lp[s]);
    M = wave_max(M);
    float L = 0.f, acc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
        const int s = s0 + lane;
        const float ls = s < nsplit ? lp[s] : -INFINITY;
        const float e = ls == -INFINITY ? 0.f : __expf(ls - M);
        L += wave_sum(e);
        const int cnt = min(64, nsplit - s0);
        const uint32_t eb = __builtin_bit_cast(uint32_t, e);
        // eight partials per batch, their loads issued together: split
        // indices past the last one re-read the last split (in bounds) and
        // take weight 0 (lanes past nsplit hold e = 0)
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            float x[8][NPL];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sj = s0 + min(j0 + j, cnt - 1);
#pragma unroll
                for (int i = 0; i < NPL; ++i) x[j][i] = op[(int64_t)sj * D + 64 * i];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float ej =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(eb, min(j0 + j, 63)));
#pragma unroll
                for (int i = 0; i < NPL; ++i) acc[i] += ej * x[j][i];
            }
        }
    }
    if (D >= 64 || lane < D) {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            o[row * D + dim + 64 * i] = (uint16_t)(pack2<DT>(acc[i] / L, 0.f) & 0xffffu);
    }
    if (lane == 0 && lse != nullptr) lse[row] = M + logf(L);
}

template <int DT, int D>
void launch_decode_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                     float* lse, float* o_part, float* lse_part, int Tq, int Tk, int nqt,
                     int nsplit, int chunk, int causal, float c, uint32_t sign, dim3 grid,
                     dim3 cgrid, int64_t rows, hipStream_t stream) {
    auto fn = causal ? decode_split16<DT, true, D> : decode_split16<DT, false, D>;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), 0, stream, q, k, v, o_part, lse_part, Tq, Tk,
                       nqt, nsplit, chunk, c, sign, (uint16_t*)nullptr, (float*)nullptr,
                       (uint32_t*)nullptr);
    hipLaunchKernelGGL((decode_combine16<DT, D>), cgrid, dim3(256), 0, stream, o_part,
                       lse_part, o, lse, rows, nsplit);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                         float* o_part, float* lse_part, int BH, int Tq, int Tk, int D,
                         int causal, float c, bool negate_q, int dt, hipStream_t stream) {
    int nsplit, chunk;
    decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    const int nqt = (Tq + kDecTile - 1) / kDecTile;
    const uint32_t sign = negate_q ? 0x80008000u : 0u;
    const dim3 grid((unsigned)(BH * nqt * nsplit));
    const int64_t rows = (int64_t)BH * Tq;
    const dim3 cgrid((unsigned)((rows + 3) / 4));
    const uint16_t* q16 = (const uint16_t*)q;
    const uint16_t* k16 = (const uint16_t*)k;
    const uint16_t* v16 = (const uint16_t*)v;
    uint16_t* o16 = (uint16_t*)o;
#define ATTN_DECODE_CASE(DTV, DV)                                                           \
    if (dt == DTV && D == DV) {                                                             \
        launch_decode_d<DTV, DV>(q16, k16, v16, o16, lse, o_part, lse_part, Tq, Tk, nqt,   \
                                 nsplit, chunk, causal, c, sign, grid, cgrid, rows, stream); \
        return hipGetLastError();                                                           \
    }
    ATTN_DECODE_CASE(ATTN_DT_BF16, 64)
    ATTN_DECODE_CASE(ATTN_DT_F16, 64)
    ATTN_DECODE_CASE(ATTN_DT_BF16, 32)
    ATTN_DECODE_CASE(ATTN_DT_F16, 32)
    ATTN_DECODE_CASE(ATTN_DT_BF16, 128)
    ATTN_DECODE_CASE(ATTN_DT_F16, 128)
#undef ATTN_DECODE_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Decode without allocation: the library's own scratch holds the per-tile
// counters (kDecodeCounters uint32, zero between calls) and, after them, the
// split partials (o_part, then lse_part). Every GPU the library runs on holds
// one copy until the process ends; calls on one GPU share it, so calls that
// overlap on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

__global__ __launch_bounds__(256) void decode_scratch_clear(uint32_t* __restrict__ counters) {
    for (int i = threadIdx.x; i < kDecodeCounters; i += 256) counters[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
unsigned char* g_scratch[kMaxDevices] = {};  // device address of scratch, per device
}  // namespace

// The device address of the current device's scratch: looked up once per
// device (hipGetSymbolAddress with that device current), when its counters
// are also cleared on `stream`; host code uses this address, never the
// array's name.
static hipError_t decode_scratch_address(unsigned char** out, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_scratch_clear, dim3(1), dim3(256), 0, stream, (uint32_t*)p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = (unsigned char*)p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

template <int DT, int D>
static void launch_decode_merged_d(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, float* o_part, float* lse_part,
                                   uint32_t* counters, int Tq, int Tk, int nqt, int nsplit,
                                   int chunk, int causal, float c, uint32_t sign, dim3 grid,
                                   hipStream_t stream) {
    auto fn = causal ? decode_split16<DT, true, D, true> : decode_split16<DT, false, D, true>;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), 0, stream, q, k, v, o_part, lse_part, Tq, Tk,
                       nqt, nsplit, chunk, c, sign, o, lse, counters);
}

size_t decode_scratch_need(int BH, int Tq, int Tk, int D) {
    int nsplit, chunk;
    decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    if (nsplit == 1) return kDecodeCounterBytes;
    const uint64_t nqt = ((uint64_t)Tq + kDecTile - 1) / kDecTile;
    if ((uint64_t)BH * nqt > (uint64_t)kDecodeCounters) return 0;
    const uint64_t parts = (uint64_t)BH * Tq * nsplit;
    return kDecodeCounterBytes + parts * (uint64_t)(D + 1) * 4;
}

hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int BH, int Tq, int Tk, int D, int causal,
                                 float c, bool negate_q, int dt, hipStream_t stream) {
    unsigned char* base = nullptr;
    hipError_t e = decode_scratch_address(&base, stream);
    if (e != hipSuccess) return e;
    int nsplit, chunk;
    decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    const int nqt = (Tq + kDecTile - 1) / kDecTile;
    const uint32_t sign = negate_q ? 0x80008000u : 0u;
    const dim3 grid((unsigned)(BH * nqt * nsplit));
    const uint64_t parts = (uint64_t)BH * Tq * nsplit;
    uint32_t* counters = (uint32_t*)base;
    float* o_part = (float*)(base + kDecodeCounterBytes);
    float* lse_part = o_part + parts * D;
    const uint16_t* q16 = (const uint16_t*)q;
    const uint16_t* k16 = (const uint16_t*)k;
    const uint16_t* v16 = (const uint16_t*)v;
    uint16_t* o16 = (uint16_t*)o;
#define ATTN_DECODE_MERGED_CASE(DTV, DV)                                                     \
    if (dt == DTV && D == DV) {                                                             \
        launch_decode_merged_d<DTV, DV>(q16, k16, v16, o16, lse, o_part, lse_part, counters, \
                                        Tq, Tk, nqt, nsplit, chunk, causal, c, sign, grid,  \
                                        stream);                                            \
        return hipGetLastError();                                                           \
    }
    ATTN_DECODE_MERGED_CASE(ATTN_DT_BF16, 64)
    ATTN_DECODE_MERGED_CASE(ATTN_DT_F16, 64)
    ATTN_DECODE_MERGED_CASE(ATTN_DT_BF16, 32)
    ATTN_DECODE_MERGED_CASE(ATTN_DT_F16, 32)
    ATTN_DECODE_MERGED_CASE(ATTN_DT_BF16, 128)
    ATTN_DECODE_MERGED_CASE(ATTN_DT_F16, 128)
#undef ATTN_DECODE_MERGED_CASE
    return hipErrorInvalidValue;
}

// Kernels 0..5 are the D = 64 ones, then D = 32 (6..11) and D = 128 (12..17),
// each group ordered bf16 {causal, full, combine}, f16 {causal, full, combine}.
template <int D>
static const void* decode_group_ptr(int index) {
    switch (index) {
        case 0: return (const void*)decode_split16<ATTN_DT_BF16, true, D>;
        case 1: return (const void*)decode_split16<ATTN_DT_BF16, false, D>;
        case 2: return (const void*)decode_combine16<ATTN_DT_BF16, D>;
        case 3: return (const void*)decode_split16<ATTN_DT_F16, true, D>;
        case 4: return (const void*)decode_split16<ATTN_DT_F16, false, D>;
        case 5: return (const void*)decode_combine16<ATTN_DT_F16, D>;
        default: return nullptr;
    }
}

const void* decode_kernel_ptr(int index) {
    if (index < 0) return nullptr;
    if (index < 6) return decode_group_ptr<64>(index);
    if (index < 12) return decode_group_ptr<32>(index - 6);
    if (index < 18) return decode_group_ptr<128>(index - 12);
    return nullptr;
}

// The merged kernels: D = 64, 32, 128, each bf16 {causal, full}, f16 {causal, full}.
template <int D>
static const void* decode_merged_group_ptr(int index) {
    switch (index) {
        case 0: return (const void*)decode_split16<ATTN_DT_BF16, true, D, true>;
        case 1: return (const void*)decode_split16<ATTN_DT_BF16, false, D, true>;
        case 2: return (const void*)decode_split16<ATTN_DT_F16, true, D, true>;
        case 3: return (const void*)decode_split16<ATTN_DT_F16, false, D, true>;
        default: return nullptr;
    }
}

const void* decode_merged_kernel_ptr(int index) {
    if (index < 0) return nullptr;
    if (index < 4) return decode_merged_group_ptr<64>(index);
    if (index < 8) return decode_merged_group_ptr<32>(index - 4);
    if (index < 12) return decode_merged_group_ptr<128>(index - 8);
    return nullptr;
}

}  // namespace attn
