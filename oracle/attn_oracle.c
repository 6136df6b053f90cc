/*
 * Attention oracle: a plain, slow, double-precision CPU evaluation of exact
 * scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark use it. It shares no
 * source, header, helper or constant with the GPU library.
 *
 * What it computes, per query row i of one (batch, head) slice:
 *
 *   visible keys J_i = {0 .. T-1}, or {0 .. i} when causal
 *       (causal mask: a token sees the tokens up to and including its own;
 *        "Flash attention in PyTorch, then in Triton", section "Attention's
 *        table of scores" and "Attention by hand")
 *   s_j   = scale * sum_e q[i,e] * k[j,e]                   for j in J_i
 *   m     = max_j s_j
 *   w_j   = exp(s_j - m),  Z = sum_j w_j                    (safe softmax)
 *   O[i,e] = (sum_j w_j * v[j,e]) / Z
 *   lse_i = m + log Z           (natural-log log-sum-exp of the scaled,
 *                                masked scores)
 *
 * The row-at-a-time, max-subtracted evaluation in double with one row of
 * scratch follows the double-precision CPU reference of the page
 * "attention.cu" (its attentionCpu function); the causal mask and the
 * log-sum-exp side output follow "Flash attention in PyTorch, then in
 * Triton" (sections "Attention by hand" and "Backwards, and training with
 * it"). The log-sum-exp is reported in natural-log units; that page keeps it
 * in base-2 units inside its kernel, which is the same quantity times log2(e).
 *
 * Inputs are float32 arrays (bf16/fp16 inputs are passed already widened to
 * float32, which is exact); every product and sum is done in double. There is
 * no blocking, no fusion and no reordering of the arithmetic: for every output
 * element the sums run over j (or e) in ascending order. Build without
 * fast-math and without floating-point contraction.
 *
 * The backward pass (oracle_attention_backward), per (batch, head) slice,
 * follows the steps of "Flash attention in PyTorch, then in Triton", section
 * "Backwards, and training with it", in that order: for an output gradient
 * dO, each row's lse and O are computed as above and delta_i = sum_e
 * dO[i,e] * O[i,e]; then for every visible pair (i, j)
 *   P_ij  = exp(s_ij - lse_i)          (the probabilities made again)
 *   dP_ij = sum_e dO[i,e] * v[j,e]
 *   dS_ij = P_ij * (dP_ij - delta_i)   (the softmax's backward)
 * and dQ_i = scale * sum_j dS_ij k_j, dK_j = scale * sum_i dS_ij q_i,
 * dV_j = sum_i P_ij dO_i, every sum ascending in its index.
 *
 * The gated linear recurrence (oracle_gated_recurrence) is the second
 * workload of the pages, the recurrence of the page "Kimi-K2.6 l2 p24"
 * (POPCORNBENCH), which has no softmax: per (batch, head) a D x D state S
 * starts at zero and, for t = 0 .. T-1 in order,
 *   S[i][j] <- gate[t][j] * S[i][j] + k[t][i] * v[t][j]     (every i, j)
 *   y[t][j]  = sum_i q[t][i] * S[i][j]                       (i ascending)
 * with q, k, v, gate and y laid out [B, T, H, D] as on that page. The gate
 * scales each column j of the state; the update comes before the readout of
 * the same step. In double, in that order, with no rearrangement.
 *
 * Parity pins (each checked by the test suite against closed forms, library
 * routines or brute force, never against this file itself):
 *   T = 1 returns V; Q = 0 returns the (prefix) mean of V; one-hot scores
 *   select one V row; probability rows sum to 1; brute force on tiny shapes;
 *   float64 scaled_dot_product_attention on small shapes; key-shift,
 *   V-affine, causal-prefix, slice-independence and permutation invariants.
 *   Backward: central differences of the forward; float64 autograd through
 *   scaled_dot_product_attention; T = 1 and Q = 0 closed forms; the key
 *   gradients sum to zero; dV does not depend on V; sum_i q_i.dQ_i equals
 *   sum_j k_j.dK_j; causal rows do not see later rows.
 *   Gated recurrence: the closed-form sum over earlier steps with gate
 *   products; gate 1 gives causal linear attention (float64 matmul); gate 0
 *   keeps only the current step; a hand-computed scalar case; causality,
 *   column and head independence, linearity in q and v.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row of one (batch, head) slice. q_row: D floats; k, v: T x D
 * floats of that slice; scratch: at least T doubles; o_row: D doubles. */
static void oracle_one_row(const float* q_row, const float* k, const float* v,
                           int64_t T, int64_t D, int causal, double scale,
                           int64_t i, double* scratch, double* o_row,
                           double* lse_out) {
    const int64_t visible = causal ? (i + 1) : T;

    /* scores and their maximum */
    double best = -INFINITY;
    for (int64_t j = 0; j < visible; ++j) {
        double dot = 0.0;
        for (int64_t e = 0; e < D; ++e) {
            dot += (double)q_row[e] * (double)k[j * D + e];
        }
        const double s = scale * dot;
        scratch[j] = s;
        if (s > best) best = s;
    }

    /* exponentials with the maximum subtracted, and their sum */
    double total = 0.0;
    for (int64_t j = 0; j < visible; ++j) {
        const double w = exp(scratch[j] - best);
        scratch[j] = w;
        total += w;
    }

    /* weighted sum of the values; for each e the sum runs over j ascending */
    for (int64_t e = 0; e < D; ++e) o_row[e] = 0.0;
    for (int64_t j = 0; j < visible; ++j) {
        const double w = scratch[j];
        const float* vj = v + j * D;
        for (int64_t e = 0; e < D; ++e) {
            o_row[e] += w * (double)vj[e];
        }
    }
    for (int64_t e = 0; e < D; ++e) o_row[e] /= total;

    if (lse_out) *lse_out = best + log(total);
}

/*
 * Attention for a set of query rows.
 *
 * q, k, v : float32, contiguous [B, H, T, D].
 * rows    : flat row ids (b * H + h) * T + t, or NULL for every row in order.
 * nrows   : number of entries of `rows` (ignored when rows is NULL).
 * o       : double [nrows, D] (or [B*H*T, D] when rows is NULL).
 * lse     : double [nrows] or NULL.
 * nthreads: OpenMP threads (<= 0: the runtime default).
 *
 * Returns 0, or -1 on invalid arguments (nothing written).
 */
int oracle_attention(const float* q, const float* k, const float* v,
                     int64_t B, int64_t H, int64_t T, int64_t D, int causal,
                     double scale, const int64_t* rows, int64_t nrows,
                     double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || H < 1 || T < 1 || D < 1) return -1;
    const int64_t all = B * H * T;
    const int64_t n = rows ? nrows : all;
    if (n < 0) return -1;
    if (rows) {
        for (int64_t r = 0; r < n; ++r) {
            if (rows[r] < 0 || rows[r] >= all) return -1;
        }
    }
    int bad = 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* scratch = (double*)malloc((size_t)T * sizeof(double));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t r = 0; r < n; ++r) {
            if (!scratch) continue;
            const int64_t flat = rows ? rows[r] : r;
            const int64_t slice = flat / T;
            const int64_t t = flat % T;
            const float* qs = q + slice * T * D;
            const float* ks = k + slice * T * D;
            const float* vs = v + slice * T * D;
            oracle_one_row(qs + t * D, ks, vs, T, D, causal, scale, t,
                           scratch, o + r * D, lse ? lse + r : NULL);
        }
        free(scratch);
    }
    (void)nthreads;
    return bad ? -2 : 0;
}

/*
 * Attention of a few new queries against a key/value cache (decode): q is
 * float32 [B, H, Tq, D], k and v are float32 [B, H, Tk, D] with Tq <= Tk.
 * Query i is the token at position Tk - Tq + i of the sequence the cache
 * holds, so with causal != 0 it sees keys 0 .. Tk - Tq + i (the mask aligned
 * to the bottom-right of the Tq x Tk table); otherwise every key. The page
 * "Flash attention in PyTorch, then in Triton" names this case (new tokens
 * against all the keys, section "Backwards, and training with it") as one
 * its kernel does not handle. Each row is oracle_one_row at that position.
 * o: double [B*H*Tq, D]; lse: double [B*H*Tq] or NULL. Returns 0, -1 on
 * invalid arguments, -2 when scratch memory could not be allocated.
 */
int oracle_attention_kv(const float* q, const float* k, const float* v,
                        int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D,
                        int causal, double scale, double* o, double* lse,
                        int nthreads) {
    if (!q || !k || !v || !o || B < 1 || H < 1 || Tq < 1 || Tk < Tq || D < 1)
        return -1;
    const int64_t n = B * H * Tq;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* scratch = (double*)malloc((size_t)Tk * sizeof(double));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t r = 0; r < n; ++r) {
            if (!scratch) continue;
            const int64_t slice = r / Tq;
            const int64_t i = r % Tq;
            oracle_one_row(q + r * D, k + slice * Tk * D, v + slice * Tk * D, Tk, D,
                           causal, scale, Tk - Tq + i, scratch, o + r * D,
                           lse ? lse + r : NULL);
        }
        free(scratch);
    }
    (void)nthreads;
    return bad ? -2 : 0;
}

/*
 * The full probability table of one head, for tiny shapes: P[i, j] is the
 * softmax weight of key j for query i (0 for a masked key). q, k: float32
 * [T, D]; P: double [T, T]. Same arithmetic as oracle_one_row.
 */
int oracle_probabilities(const float* q, const float* k, int64_t T, int64_t D,
                         int causal, double scale, double* P) {
    if (!q || !k || !P || T < 1 || D < 1) return -1;
    for (int64_t i = 0; i < T; ++i) {
        const int64_t visible = causal ? (i + 1) : T;
        double* row = P + i * T;
        double best = -INFINITY;
        for (int64_t j = 0; j < visible; ++j) {
            double dot = 0.0;
            for (int64_t e = 0; e < D; ++e) {
                dot += (double)q[i * D + e] * (double)k[j * D + e];
            }
            row[j] = scale * dot;
            if (row[j] > best) best = row[j];
        }
        double total = 0.0;
        for (int64_t j = 0; j < visible; ++j) {
            row[j] = exp(row[j] - best);
            total += row[j];
        }
        for (int64_t j = 0; j < visible; ++j) row[j] /= total;
        for (int64_t j = visible; j < T; ++j) row[j] = 0.0;
    }
    return 0;
}

/* s_ij = scale * q_i . k_j, P_ij = exp(s_ij - lse_i), dP_ij = dO_i . v_j and
 * dS_ij = P_ij * (dP_ij - delta_i) for one visible pair (i, j < T) of one
 * slice (q, k, v, dout: float32 [T, D] of the slice). */
static void oracle_pair(const float* q, const float* k, const float* v,
                        const float* dout, int64_t T, int64_t D, double scale,
                        const double* lse, const double* delta, int64_t i,
                        int64_t j, double* P, double* dS) {
    double dot = 0.0, dpv = 0.0;
    (void)T;
    for (int64_t e = 0; e < D; ++e) dot += (double)q[i * D + e] * (double)k[j * D + e];
    for (int64_t e = 0; e < D; ++e) dpv += (double)dout[i * D + e] * (double)v[j * D + e];
    *P = exp(scale * dot - lse[i]);
    *dS = *P * (dpv - delta[i]);
}

/*
 * Gradients of attention for whole (batch, head) slices.
 *
 * q, k, v, dout : float32, contiguous [B, H, T, D] (dout = dL/dO).
 * slices        : slice ids b * H + h, or NULL for every slice in order.
 * nslices       : number of entries of `slices` (ignored when NULL).
 * dq, dk, dv    : double [nslices, T, D] (or [B*H, T, D] when slices is NULL).
 * nthreads      : OpenMP threads (<= 0: the runtime default).
 *
 * Returns 0, -1 on invalid arguments (nothing written), -2 when scratch
 * memory could not be allocated.
 */
int oracle_attention_backward(const float* q, const float* k, const float* v,
                              const float* dout, int64_t B, int64_t H,
                              int64_t T, int64_t D, int causal, double scale,
                              const int64_t* slices, int64_t nslices,
                              double* dq, double* dk, double* dv,
                              int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 1 || H < 1 ||
        T < 1 || D < 1)
        return -1;
    const int64_t n = slices ? nslices : B * H;
    if (n < 0) return -1;
    if (slices) {
        for (int64_t r = 0; r < n; ++r) {
            if (slices[r] < 0 || slices[r] >= B * H) return -1;
        }
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#endif
    double* lse = (double*)malloc((size_t)T * sizeof(double));
    double* delta = (double*)malloc((size_t)T * sizeof(double));
    if (!lse || !delta) {
        free(lse);
        free(delta);
        return -2;
    }
    int bad = 0;
    for (int64_t r = 0; r < n && !bad; ++r) {
        const int64_t slice = slices ? slices[r] : r;
        const float* qs = q + slice * T * D;
        const float* ks = k + slice * T * D;
        const float* vs = v + slice * T * D;
        const float* ds = dout + slice * T * D;
        double* dqs = dq + r * T * D;
        double* dks = dk + r * T * D;
        double* dvs = dv + r * T * D;

        /* each row's lse and O, and delta_i = dO_i . O_i */
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
#endif
        {
            double* scratch = (double*)malloc((size_t)T * sizeof(double));
            double* o_row = (double*)malloc((size_t)D * sizeof(double));
            if (!scratch || !o_row) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
                bad = 1;
            }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (int64_t i = 0; i < T; ++i) {
                if (!scratch || !o_row) continue;
                oracle_one_row(qs + i * D, ks, vs, T, D, causal, scale, i,
                               scratch, o_row, &lse[i]);
                double d = 0.0;
                for (int64_t e = 0; e < D; ++e) d += (double)ds[i * D + e] * o_row[e];
                delta[i] = d;
            }
            free(scratch);
            free(o_row);
        }
        if (bad) break;

        /* dQ_i = scale * sum_j dS_ij k_j, j ascending */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
#endif
        for (int64_t i = 0; i < T; ++i) {
            const int64_t visible = causal ? (i + 1) : T;
            double* g = dqs + i * D;
            for (int64_t e = 0; e < D; ++e) g[e] = 0.0;
            for (int64_t j = 0; j < visible; ++j) {
                double P, dS;
                oracle_pair(qs, ks, vs, ds, T, D, scale, lse, delta, i, j, &P, &dS);
                for (int64_t e = 0; e < D; ++e) g[e] += dS * (double)ks[j * D + e];
            }
            for (int64_t e = 0; e < D; ++e) g[e] *= scale;
        }

        /* dK_j = scale * sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i, i
         * ascending over the queries that see key j */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
#endif
        for (int64_t j = 0; j < T; ++j) {
            double* gk = dks + j * D;
            double* gv = dvs + j * D;
            for (int64_t e = 0; e < D; ++e) gk[e] = gv[e] = 0.0;
            for (int64_t i = causal ? j : 0; i < T; ++i) {
                double P, dS;
                oracle_pair(qs, ks, vs, ds, T, D, scale, lse, delta, i, j, &P, &dS);
                for (int64_t e = 0; e < D; ++e) {
                    gk[e] += dS * (double)qs[i * D + e];
                    gv[e] += P * (double)ds[i * D + e];
                }
            }
            for (int64_t e = 0; e < D; ++e) gk[e] *= scale;
        }
    }
    free(lse);
    free(delta);
    (void)nthreads;
    return bad ? -2 : 0;
}

/* The gated linear recurrence above, for every (batch, head); inputs
 * float32 [B, T, H, D], output y double [B, T, H, D]. Returns 0, or -1 for
 * invalid sizes or an allocation failure. */
int oracle_gated_recurrence(const float* q, const float* k, const float* v,
                            const float* gate, int64_t B, int64_t T, int64_t H,
                            int64_t D, double* y, int nthreads) {
    if (B < 1 || T < 1 || H < 1 || D < 1) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        double* S = (double*)calloc((size_t)(D * D), sizeof(double));
        if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = ((b * T + t) * H + h) * D;
            for (int64_t i = 0; i < D; ++i)
                for (int64_t j = 0; j < D; ++j)
                    S[i * D + j] = (double)gate[row + j] * S[i * D + j] +
                                   (double)k[row + i] * (double)v[row + j];
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < D; ++i) acc += (double)q[row + i] * S[i * D + j];
                y[row + j] = acc;
            }
        }
        free(S);
    }
    (void)nthreads;
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use by default. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
