// The online-softmax step of the 16-bit forward kernels for gfx950, shared
// by every head dimension: one 64-key tile of S^T in two 32x32 accumulators
// (lane = query row, register r = key row acc_row(r, lane half)), a running
// reference maximum, and O^T in NO 32-dim accumulators.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fused_layout.h"
#include "gfx950.h"

namespace attn {

// Lazy rescaling. The online softmax may exponentiate against any reference
// point m, as long as O, l and lse all use the same one and no weight
// overflows. A tile whose row maximum exceeds the reference by at most
// kLazyLog2 (in log2 units, so every weight is <= 2^kLazyLog2 = 256) is
// exponentiated against the old reference; only a larger jump moves the
// reference and rescales O and l by exp2(m_old - m_new). After the first
// tile this is rare for typical scores, and the decision is wave-uniform.
constexpr float kLazyLog2 = 8.0f;

// Online-softmax state of one lane: the reference maximum m (raw score
// units), mc = m * c, and this lane-half's running denominator l.
struct RowState {
    float m, mc, l;
};

// The online-softmax step of one tile: the weights p = exp2(s*c - m*c)
// rounded into the P fragment and their sum into l, with the lazy reference
// update (O and l rescaled by exp2(m_old - m_new) when some row's maximum
// jumps by more than kLazyLog2). EDGE tiles (keys >= T and, causal, keys
// after the row, set to -inf) take the row maximum first. Unmasked tiles
// take the weights first against the current reference and need no
// maximum: a lane's 32 weights are each at most their sum t, so t <= 2^8 in
// every lane keeps every weight within the bound (an overflow to inf fails
// the test too); otherwise (rare) the maximum is taken, the reference moved
// if it jumped by more than kLazyLog2, and the weights made again from S,
// which is still in registers. Both orders take the same decisions, so
// the results are the same bits.
//
// `pending` is work that must reach O before any rescale of it (the previous
// tile's P.V products in a skewed loop): it runs first, and on unmasked
// tiles in the same block as the weights, so its matrix instructions can
// issue between the weights' vector instructions.
struct NoPending {
    __device__ void operator()() const {}
};
template <int DT, bool CAUSAL, bool EDGE, int NO, typename Pending = NoPending>
__device__ inline void softmax_tile(v16f32 (&s)[2], v4u32 (&pf)[4],
                                    v16f32 (&oacc)[NO], RowState& st, float c,
                                    int k0, int T, int my_q, int hh,
                                    Pending pending = Pending()) {
    auto weights = [&](float mc) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int nt = ks >> 1, r0 = (ks & 1) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = s[nt][r0 + 2 * i], x1 = s[nt][r0 + 2 * i + 1];
                float p0 = fast_exp2(fmaf(x0, c, -mc));
                float p1 = fast_exp2(fmaf(x1, c, -mc));
                if (EDGE) {
                    if (x0 == -INFINITY) p0 = 0.f;
                    if (x1 == -INFINITY) p1 = 0.f;
                }
                pf[ks][i] = pack2<DT>(p0, p1);
                if (i & 1)
                    t1 = sum2<DT>(pf[ks][i], t1);
                else
                    t0 = sum2<DT>(pf[ks][i], t0);
            }
        }
        return t0 + t1;
    };
    auto rescale = [&]() {
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
            for (int mt = 0; mt < NO; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[mt][r] *= corr;
        }
    };
    if (EDGE) {
        pending();
        // key k0 + 32 nt + acc_row(r, hh) is masked when it is past T - 1 or
        // (causal) past the row: with lim = min(T - 1, row) - k0 - 4 hh that
        // is 32 nt + acc_row(r, 0) > lim, a constant against one per-lane
        // value (no per-register offsets kept live across the loop)
        int lim = (CAUSAL ? min(T - 1, my_q) : T - 1) - k0 - 4 * hh;
        asm("" : "+v"(lim));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * nt + acc_row(r, 0) > lim) s[nt][r] = -INFINITY;
        rescale();
        st.l += weights(st.mc);
    } else {
        pending();
        float t = weights(st.mc);
        if (__builtin_amdgcn_ballot_w64(!(t <= 256.0f)) != 0) {
            rescale();
            t = weights(st.mc);
        }
        st.l += t;
    }
}

}  // namespace attn
