/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention forward library
 * (libattn.so).
 *
 * The operation is exact scaled-dot-product attention (head dimension 64 on
 * every path; 32 and 128 also on the 16-bit fused forward),
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:] . k[b,h,j,:] ) v[b,h,j,:]
 *
 * over the keys j visible to query i (all j < T, or j <= i when causal), plus
 * the per-row log-sum-exp  lse[b,h,i] = log sum_j exp(scale * q_i . k_j)  in
 * natural-log units. Definitions: "Flash attention in PyTorch, then in
 * Triton", section "Attention's table of scores" (scores, causal mask,
 * softmax, weighted values) and section "Backwards, and training with it"
 * (the per-row log-sum-exp the forward pass keeps). The fused path computes it
 * the way that page's section "Flash attention" describes (the online
 * softmax: key tiles with a running maximum, denominator and output, rescaled
 * when a larger maximum arrives), so the T x T score table never exists. The
 * naive path is the materialising contrast of the page "attention.cu" (a
 * tiled Q K^T into a T x T buffer, a max pass and an exp-and-sum pass into a
 * second buffer, then a tiled P V divided by the row sums).
 *
 * Conventions shared by every entry point:
 *  - Layout: q, k, v, o are contiguous row-major [B, H, T, D] arrays of the
 *    element type `dtype` (element (b,h,t,e) at ((b*H + h)*T + t)*D + e);
 *    lse is a contiguous float32 [B, H, T] array.
 *  - Memory: q, k, v, o, lse, workspace are DEVICE pointers on the current
 *    HIP device. The caller owns every buffer; the library allocates nothing
 *    and keeps no pointer after the call returns.
 *  - Alignment: q, k, v, o and workspace must be 16-byte aligned (the kernels
 *    use 128-bit accesses); lse must be 4-byte aligned.
 *  - Streams: `stream` is a hipStream_t (NULL means the null stream). Calls
 *    return once the work is enqueued; the results are ready after the
 *    stream is synchronised. A fault inside a kernel surfaces at that
 *    synchronisation, not as a return code.
 *  - Errors: every entry point returns an attn_status. Arguments are checked
 *    before any HIP call, so an invalid call has no side effect and touches
 *    no device. The library never prints and never exits.
 *  - Threads: calls are re-entrant; attn_last_hip_error() is per thread.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. lse is always float32. */
typedef enum {
    ATTN_F32 = 0,  /* float32; products on the fp32 matrix cores          */
    ATTN_BF16 = 1, /* bfloat16 in, float32 accumulate, bfloat16 out       */
    ATTN_F16 = 2   /* float16 in, float32 accumulate, float16 out         */
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = -1,     /* a null or misaligned pointer, a size < 1,
                                  an unknown dtype, a non-finite scale, a
                                  workspace too small, a null output struct */
    ATTN_ERR_UNSUPPORTED = -2, /* a well-formed request this library does not
                                  implement: a head dimension the path has
                                  no kernel for, a non-fp32 naive call,
                                  a grid larger than one launch holds, or a
                                  16-bit slice over 4 GiB                    */
    ATTN_ERR_HIP = -3          /* the HIP runtime refused a launch or query;
                                  the code is kept for attn_last_hip_error() */
} attn_status;

typedef enum { ATTN_PATH_FUSED = 0, ATTN_PATH_NAIVE = 1 } attn_path;

/*
 * attn_fwd_stream - fused attention forward (online softmax, no T x T table).
 *
 * q, k, v : device, [B, H, T, D] of `dtype`, read only.
 * o       : device, [B, H, T, D] of `dtype`, written (every element).
 * lse     : device, float32 [B, H, T], written; may be NULL to skip it.
 * B, H, T : batch, heads, tokens; each >= 1. Queries and keys share T.
 * D       : head dimension: 64, or 32 or 128 for bf16 / f16 (one kernel is
 *           built per head dimension, the way the pages' own kernels take it
 *           as a compile-time constant); ATTN_ERR_UNSUPPORTED otherwise.
 * causal  : nonzero => key j is visible to query i iff j <= i (top-left
 *           aligned); zero => every key is visible.
 * scale   : multiplies q . k before the softmax (usually 1/sqrt(D)); any
 *           finite value, including 0 and negative values.
 * dtype   : an attn_dtype.
 * stream  : hipStream_t or NULL.
 *
 * Returns ATTN_OK once enqueued, or an error status with nothing enqueued;
 * ATTN_ERR_UNSUPPORTED also for a 16-bit dtype with T * D * 2 > 2^32 - 1
 * bytes per (batch, head) slice (one K or V slice is addressed as a single
 * buffer).
 * Extra device memory: none (the caller's lse is the only O(T) side output).
 * The kernel launched depends on dtype, D and the grid size
 * (attn_fused_kernel names it); every kernel computes the same result to
 * rounding.
 */
int attn_fwd_stream(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int T, int D, int causal,
                    float scale, int dtype, void* stream);

/* attn_fwd - attn_fwd_stream on the null stream. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int T, int D, int causal, float scale, int dtype);

/*
 * attn_naive_fwd - the materialising contrast path, float32 only.
 *
 * Same meaning for q, k, v, o, lse, B, H, T, D, causal, scale and stream as
 * attn_fwd_stream (lse may be NULL). workspace is a caller-owned device
 * buffer of at least attn_naive_workspace_bytes(B, H, T) bytes; it receives
 * the score table S [B,H,T,T], the exponential table P [B,H,T,T] and the row
 * sums [B,H,T], all float32, and its contents are undefined afterwards.
 * Returns ATTN_ERR_UNSUPPORTED for dtype != ATTN_F32 (the dtype argument is
 * part of the signature so the two paths take the same arguments).
 */
int attn_naive_fwd(const float* q, const float* k, const float* v, float* o,
                   float* lse, void* workspace, size_t workspace_bytes, int B,
                   int H, int T, int D, int causal, float scale, int dtype,
                   void* stream);

/* Workspace bytes attn_naive_fwd needs: (2*B*H*T*T + B*H*T) * 4 rounded up
 * to 256 bytes; 0 for sizes < 1 or when the count overflows 64 bits. */
size_t attn_naive_workspace_bytes(int B, int H, int T);

/*
 * attn_bwd_stream - gradients of attention with respect to q, k and v (the
 * backward pass of "Flash attention in PyTorch, then in Triton", section
 * "Backwards, and training with it"): with P rebuilt from the scores and
 * the forward's lse, delta = rowsum(dO * O), dS = P (dO V^T - delta),
 *   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
 *
 * q, k, v   : device, [B, H, T, D] of `dtype`, the forward's inputs.
 * o, lse    : device, the forward's output ([B, H, T, D] of `dtype`) and
 *             log-sum-exp (float32 [B, H, T], natural log), as attn_fwd
 *             wrote them for the same causal and scale.
 * dout      : device, [B, H, T, D] of `dtype`: dL/dO.
 * dq, dk, dv: device, [B, H, T, D] of `dtype`, written (every element);
 *             accumulated in float32, rounded to nearest even once.
 * workspace : caller-owned device buffer of at least
 *             attn_bwd_workspace_bytes(B, H, T) bytes (16-byte aligned); it
 *             receives -delta and lse * log2(e) of every row (float32);
 *             contents undefined after.
 * B, H, T, D, causal, scale, stream: as in attn_fwd_stream.
 * dtype     : ATTN_BF16 or ATTN_F16; ATTN_F32 returns ATTN_ERR_UNSUPPORTED.
 *
 * Returns ATTN_OK once enqueued, or an error status with nothing enqueued:
 * ATTN_ERR_INVALID for a null pointer, a pointer not 16-byte aligned (lse: 4),
 * a bad size or dtype, a non-finite scale or a short workspace;
 * ATTN_ERR_UNSUPPORTED for D != 64, float32, or a grid or slice too large.
 * Extra device memory: the caller's workspace only.
 */
int attn_bwd_stream(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int T,
                    int D, int causal, float scale, int dtype, void* stream);

/* Workspace bytes attn_bwd_stream needs: two float32 values per row (delta
 * and the scaled lse), 2 * 4 * B*H*T with B*H*T rounded up to a multiple of
 * 64; 0 for sizes < 1 or when the count overflows 64 bits. */
size_t attn_bwd_workspace_bytes(int B, int H, int T);

/*
 * attn_bwd_atomic_stream - the same gradients as attn_bwd_stream (same
 * arguments, same definition: "Flash attention in PyTorch, then in Triton",
 * section "Backwards, and training with it"), computed with one main kernel
 * per key block that makes S, P, dP and dS once and adds each block's share
 * of dQ = scale dS K into a float32 copy of dQ with atomic adds; a last
 * kernel rounds that copy into dq.
 *
 * workspace : caller-owned device buffer of at least
 *             attn_bwd_atomic_workspace_bytes(B, H, T) bytes (16-byte
 *             aligned): delta (float32 [B, H, T], padded to 256 bytes), then
 *             the float32 dQ copy ([B, H, T, D]); zeroed by the call itself,
 *             contents undefined after.
 * dk, dv    : summed in one fixed order per element, as attn_bwd_stream.
 * dq        : float32 sums in an order the atomics decide, so two calls may
 *             differ in the last bits (within the same error bound).
 *
 * Returns and errors as attn_bwd_stream. Extra device memory: the caller's
 * workspace only.
 */
int attn_bwd_atomic_stream(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int T,
                           int D, int causal, float scale, int dtype, void* stream);

/* Workspace bytes attn_bwd_atomic_stream needs: attn_bwd_workspace_bytes(B,
 * H, T) + B*H*T*64*4; 0 for sizes < 1 or when the count overflows 64 bits. */
size_t attn_bwd_atomic_workspace_bytes(int B, int H, int T);

/*
 * attn_decode_stream - attention of Tq new queries against a key/value cache
 * of Tk tokens (decode). Query i is the token at position Tk - Tq + i, so
 * with causal != 0 it sees keys 0 .. Tk - Tq + i (the mask aligned to the
 * bottom-right of the Tq x Tk table); otherwise every key. "Flash attention
 * in PyTorch, then in Triton" (section "Backwards, and training with it")
 * names this case as one its kernel does not handle.
 *
 * q         : device, [B, H, Tq, D] of `dtype`, read only.
 * k, v      : device, [B, H, Tk, D] of `dtype`, read only (the cache).
 * o         : device, [B, H, Tq, D] of `dtype`, written.
 * lse       : device, float32 [B, H, Tq] (natural log), written; may be NULL.
 * workspace : caller-owned device buffer of at least
 *             attn_decode_workspace_bytes(B, H, Tq, Tk, D) bytes (16-byte
 *             aligned) for the per-split partial results; contents undefined
 *             afterwards.
 * Tq, Tk    : 1 <= Tq <= Tk. D is 32, 64 or 128. scale, stream as
 *             attn_fwd_stream.
 * dtype     : ATTN_BF16 or ATTN_F16; ATTN_F32 returns ATTN_ERR_UNSUPPORTED.
 *
 * The keys are split over workgroups and the partial results merged with the
 * log-sum-exp identity O = sum_s exp(lse_s - lse) O_s. Returns ATTN_OK once
 * enqueued, or an error status with nothing enqueued (ATTN_ERR_INVALID for a
 * null or misaligned pointer, Tq > Tk, a bad size, dtype or scale, a short
 * workspace; ATTN_ERR_UNSUPPORTED for another D, float32, or sizes beyond
 * one launch or a 4 GiB slice).
 */
int attn_decode_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int B, int H, int Tq,
                       int Tk, int D, int causal, float scale, int dtype, void* stream);

/* Workspace bytes attn_decode_stream needs for these sizes (the split is
 * chosen from them): about B*H*Tq*nsplit*(D + 1)*4, nsplit the number of key
 * ranges; 0 for invalid sizes, a head dimension other than 32, 64 or 128, or
 * on overflow. */
size_t attn_decode_workspace_bytes(int B, int H, int Tq, int Tk, int D);

/*
 * attn_decode_noalloc_stream - attn_decode_stream without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). It allocates
 * nothing and calls no allocating routine: the split partials and one
 * counter per (batch, head, 32-query tile) live in the library's own static
 * device scratch of ATTN_DECODE_SCRATCH_BYTES (4.03 MiB; each GPU the library
 * runs on holds one copy until the process ends), and the last workgroup of
 * each tile to finish merges the partials itself, so the call is one kernel
 * launch (two on a device's first call, which also clears the counters).
 *
 * Arguments, layouts and results are those of attn_decode_stream minus the
 * workspace. Every call on one GPU uses that GPU's one scratch: calls that
 * overlap on one GPU (concurrent streams or host threads) race and must be
 * serialised by the caller. The counters are back at zero when a call ends.
 * Returns ATTN_OK once enqueued, or an error status with nothing enqueued:
 * the errors of attn_decode_stream, and ATTN_ERR_UNSUPPORTED when the sizes
 * need more scratch than ATTN_DECODE_SCRATCH_BYTES (more than 256 tiles
 * with the keys split, which the split plan never chooses).
 */
#define ATTN_DECODE_SCRATCH_BYTES 4228096u
int attn_decode_noalloc_stream(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int H, int Tq, int Tk, int D, int causal,
                               float scale, int dtype, void* stream);

/*
 * attn_gated_recurrence_stream - the gated linear recurrence of the
 * POPCORNBENCH transcript "Kimi-K2.6 l2 p24" (no softmax): per (batch,
 * head) a D x D state S starts at zero and, for t = 0 .. T-1 in order,
 *   S[i][j] <- gate[t][j] * S[i][j] + k[t][i] * v[t][j]   (every i, j)
 *   y[t][j]  = sum_i q[t][i] * S[i][j].
 *
 * q, k, v, gate : device, float32 [B, T, H, D] (element (b,t,h,e) at
 *                 ((b*T + t)*H + h)*D + e, the page's layout), read only.
 * y             : device, float32 [B, T, H, D], written (every element).
 * B, T, H, D    : each >= 1; D <= 64 and T * H * D * 4 < 2^31 bytes
 *                 (ATTN_ERR_UNSUPPORTED beyond).
 * stream        : hipStream_t or NULL.
 * Pointers need 4-byte alignment. No workspace: the state lives in
 * registers. Returns ATTN_OK once enqueued, or an error status with nothing
 * enqueued.
 */
int attn_gated_recurrence_stream(const float* q, const float* k, const float* v,
                                 const float* gate, float* y, int B, int T, int H, int D,
                                 void* stream);

/* Arithmetic convention for the recurrence: per step and state element a
 * product k v, a multiply-add for the gate and a multiply-add for the
 * readout, 5 flops, so 5 B T H D^2; 0 for sizes < 1. */
double attn_gated_recurrence_flops(int B, int T, int H, int D);

/* Arithmetic convention for the backward pass: five products to the
 * forward's two (dP, dV, dQ, dK and the recomputed scores), so 2.5 times
 * attn_flops ("Flash attention in PyTorch, then in Triton", section
 * "Backwards, and training with it"); the two-kernel split computes the
 * scores and dP twice, which this count does not credit. */
double attn_bwd_flops(int B, int H, int T, int D, int causal);

/*
 * Memory traffic of one call, as arithmetic (no device is touched). The
 * page "attention.cu" prints these counts before any time is measured.
 *
 *   floor        : Q, K, V read once and O written once, plus the lse row
 *                  values (4 bytes per row) - the least any exact path moves.
 *   ask          : bytes the path's kernels request from global memory as
 *                  launched (fused: Q once, O and lse once, and K and V once
 *                  per query tile that reads them; naive: see below). Whether
 *                  a request reaches DRAM or hits a cache is not modelled.
 *   score_matrix : naive only - bytes spent on the T x T tables: S written,
 *                  S read twice, P written, P read once (5 passes of
 *                  4*T*T bytes per head); 0 for the fused path.
 *   table_bytes  : naive only - bytes of device memory the tables occupy
 *                  (the workspace); 0 for the fused path.
 */
typedef struct {
    uint64_t floor;
    uint64_t ask;
    uint64_t score_matrix;
    uint64_t table_bytes;
} attn_traffic;

int attn_traffic_bytes(int path, int B, int H, int T, int D, int dtype,
                       int causal, attn_traffic* out);

/* Arithmetic convention for throughput: each of the two products costs
 * 2*T*T*D flops per head (a multiply and an add), with half the table
 * masked away when causal: 4*B*H*T*T*D non-causal, 2*B*H*T*T*D causal
 * ("Flash attention in PyTorch, then in Triton", section "Attention by
 * hand"). Returned as a double; 0 for sizes < 1. */
double attn_flops(int B, int H, int T, int D, int causal);

/* Static text for a status code (never NULL). */
const char* attn_status_string(int status);

/* The hipError_t of the calling thread's last ATTN_ERR_HIP (0 if none). */
int attn_last_hip_error(void);

/*
 * Per-kernel resource figures from the HIP runtime (registers, LDS, resident
 * workgroups per compute unit), the same table "attention.cu" prints from
 * its runtime API. kernel ranges over [0, attn_kernel_count()). Needs a GPU;
 * returns ATTN_ERR_HIP without one.
 */
typedef struct {
    int num_regs;              /* vector registers per lane               */
    int lds_bytes;             /* static LDS per workgroup                */
    int private_bytes;         /* per-lane scratch (spills); 0 is healthy */
    int threads_per_workgroup; /* launch width used by the library        */
    int workgroups_per_cu;     /* occupancy API, at that width            */
} attn_kernel_attr;

int attn_kernel_count(void);
const char* attn_kernel_name(int kernel);
int attn_kernel_attributes(int kernel, attn_kernel_attr* out);

/* Tile geometry of the fused path, for traffic arithmetic and tests:
 * queries per workgroup and keys per LDS tile for `dtype`. A float32 call
 * whose grid would have fewer than 256 such workgroups (B*H*ceil(T/128))
 * runs a kernel that splits the keys among the waves of a workgroup of 32
 * query rows instead. A 16-bit call with D = 64 runs the eight-wave kernel
 * on 256 query rows per workgroup when full with B*H*ceil(T/256) >= 256,
 * or causal with B*H*(ceil(T/256) + 1) >= 600; other causal calls, and
 * full calls with B*H*ceil(T/128) <= 256, run its key-split form (128
 * query rows per workgroup, the key tiles shared out between two groups of
 * waves). attn_traffic_bytes counts the tiles of the kernel that runs. */
int attn_fused_tile(int dtype, int* block_m, int* block_n);

/* The kernel attn_fwd / attn_fwd_stream launch for these arguments, as an
 * index into the kernel table (attn_kernel_name, attn_kernel_attributes),
 * or the negative status attn_fwd would return for them (shape and dtype
 * checks only; no pointer is involved). Host-only, no GPU needed. */
int attn_fused_kernel(int B, int H, int T, int D, int causal, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
