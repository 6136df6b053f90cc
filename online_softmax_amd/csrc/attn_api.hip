// The C ABI (include/attn.h): argument validation, dispatch to the kernels,
// traffic arithmetic and runtime queries. Every check runs before the first
// HIP call, so invalid calls are side-effect free and testable without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn.h"
#include "fused_layout.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool valid_dtype(int dtype) {
    return dtype == ATTN_F32 || dtype == ATTN_BF16 || dtype == ATTN_F16;
}

// 64-bit product with overflow detection (all operands >= 0).
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > UINT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Head dimensions the 16-bit forward and decode kernels are built for; every
// other path (float32 forward, naive, backward) takes 64 only.
bool fwd16_head_dim(int D) { return D == 32 || D == attn::kHeadDim || D == 128; }

// Shape checks shared by every path, for a head dimension the caller
// accepts (`dim_ok`). Returns ATTN_OK or an error status.
int check_shape(int B, int H, int T, int D, bool dim_ok) {
    if (B < 1 || H < 1 || T < 1 || D < 1) return ATTN_ERR_INVALID;
    if (!dim_ok) return ATTN_ERR_UNSUPPORTED;
    uint64_t bh, elems;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || bh > (uint64_t)INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    if (!mul_ok(bh * (uint64_t)T, (uint64_t)D, &elems)) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

// Largest 1-D grid one fused launch takes: workgroups * 512 threads must
// stay below 2^32.
constexpr uint64_t kMaxFusedWorkgroups = (1ull << 23) - 1;

// Largest head dimension of the gated recurrence (8 state rows per lane).
constexpr int kMaxRecurrenceDim = 64;

}  // namespace

extern "C" {

int attn_fwd_stream(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int T, int D, int causal,
                    float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    int st = check_shape(B, H, T, D,
                         dtype == ATTN_F32 ? D == attn::kHeadDim : fwd16_head_dim(D));
    if (st != ATTN_OK) return st;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return ATTN_ERR_INVALID;
    if (lse && !aligned4(lse)) return ATTN_ERR_INVALID;
    int bm, bn;
    attn_fused_tile(dtype, &bm, &bn);
    const uint64_t nq = ((uint64_t)T + bm - 1) / bm;
    if (nq * (uint64_t)B * (uint64_t)H > kMaxFusedWorkgroups)
        return ATTN_ERR_UNSUPPORTED;
    // the 16-bit kernel addresses one (batch, head) slice of K or V through a
    // buffer resource with a 32-bit byte size
    if (dtype != ATTN_F32 && (uint64_t)T * D * 2 > UINT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    // exp2 multiplier: |scale| * log2(e); a negative scale negates Q instead
    const double c = fabs((double)scale) * 1.4426950408889634073599;
    if (!isfinite((float)c)) return ATTN_ERR_INVALID;
    const hipError_t e =
        D == attn::kHeadDim
            ? attn::launch_fused(q, k, v, o, lse, B * H, T, causal ? 1 : 0, (float)c,
                                 scale < 0.0f, dtype, (hipStream_t)stream)
            : attn::launch_fused_hd(q, k, v, o, lse, B * H, T, D, causal ? 1 : 0,
                                    (float)c, scale < 0.0f, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int T, int D, int causal, float scale, int dtype) {
    return attn_fwd_stream(q, k, v, o, lse, B, H, T, D, causal, scale, dtype,
                           nullptr);
}

// Two float32 arrays of one value per row (-delta, lse * log2(e)), each
// starting on a 256-byte boundary (bwd_ws_stride).
size_t attn_bwd_workspace_bytes(int B, int H, int T) {
    if (B < 1 || H < 1 || T < 1) return 0;
    uint64_t bh, rows, bytes;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh)) return 0;
    if (!mul_ok(bh, (uint64_t)T, &rows)) return 0;
    if (rows > ((uint64_t)1 << 60)) return 0;
    if (!mul_ok((uint64_t)attn::bwd_ws_stride((long long)rows), 8, &bytes)) return 0;
    return (size_t)bytes;
}

int attn_bwd_stream(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int T,
                    int D, int causal, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
        return ATTN_ERR_INVALID;
    int st = check_shape(B, H, T, D, D == attn::kHeadDim);
    if (st != ATTN_OK) return st;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    const void* p16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : p16)
        if (!aligned16(p)) return ATTN_ERR_INVALID;
    if (!aligned4(lse)) return ATTN_ERR_INVALID;
    const size_t need = attn_bwd_workspace_bytes(B, H, T);
    if (need == 0) return ATTN_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return ATTN_ERR_INVALID;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t nkb = ((uint64_t)T + attn::kBwdBlockKV - 1) / attn::kBwdBlockKV;
    const uint64_t nq = ((uint64_t)T + attn::kBlockM - 1) / attn::kBlockM;
    if (nkb * bh > kMaxFusedWorkgroups || nq * bh > kMaxFusedWorkgroups ||
        (bh * T + 31) / 32 > (uint64_t)INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    if ((uint64_t)T * D * 2 > UINT32_MAX) return ATTN_ERR_UNSUPPORTED;
    const double c = fabs((double)scale) * 1.4426950408889634073599;
    if (!isfinite((float)c)) return ATTN_ERR_INVALID;
    const hipError_t e = attn::launch_bwd(q, k, v, o, dout, lse, dq, dk, dv,
                                          (float*)workspace, B * H, T, causal ? 1 : 0,
                                          (float)c, scale, scale < 0.0f, dtype,
                                          (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

size_t attn_bwd_atomic_workspace_bytes(int B, int H, int T) {
    const size_t rows = attn_bwd_workspace_bytes(B, H, T);
    if (rows == 0) return 0;
    uint64_t bh, elems, bytes;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh)) return 0;
    if (!mul_ok(bh * (uint64_t)T, (uint64_t)attn::kHeadDim, &elems)) return 0;
    if (!mul_ok(elems, 4, &bytes)) return 0;
    if (bytes > UINT64_MAX - rows) return 0;
    return (size_t)(rows + bytes);
}

int attn_bwd_atomic_stream(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int T,
                           int D, int causal, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
        return ATTN_ERR_INVALID;
    int st = check_shape(B, H, T, D, D == attn::kHeadDim);
    if (st != ATTN_OK) return st;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    const void* p16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : p16)
        if (!aligned16(p)) return ATTN_ERR_INVALID;
    if (!aligned4(lse)) return ATTN_ERR_INVALID;
    const size_t need = attn_bwd_atomic_workspace_bytes(B, H, T);
    if (need == 0) return ATTN_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return ATTN_ERR_INVALID;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t nkb = ((uint64_t)T + attn::kBwdBlockKV - 1) / attn::kBwdBlockKV;
    // grids: key blocks; 32 rows per workgroup (prep); 2048 values per
    // workgroup (finish)
    if (nkb * bh > kMaxFusedWorkgroups || (bh * T + 31) / 32 > (uint64_t)INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    if ((uint64_t)T * D * 2 > UINT32_MAX) return ATTN_ERR_UNSUPPORTED;
    const double c = fabs((double)scale) * 1.4426950408889634073599;
    if (!isfinite((float)c)) return ATTN_ERR_INVALID;
    const size_t delta_bytes = attn_bwd_workspace_bytes(B, H, T);
    float* delta = (float*)workspace;
    float* dq_acc = (float*)((char*)workspace + delta_bytes);
    const hipError_t e = attn::launch_bwd_atomic(q, k, v, o, dout, lse, dq, dk, dv, delta,
                                                 dq_acc, B * H, T, causal ? 1 : 0, (float)c,
                                                 scale, scale < 0.0f, dtype,
                                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

size_t attn_decode_workspace_bytes(int B, int H, int Tq, int Tk, int D) {
    if (B < 1 || H < 1 || Tq < 1 || Tk < Tq || !fwd16_head_dim(D)) return 0;
    uint64_t bh, rows;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || bh > (uint64_t)INT32_MAX) return 0;
    if (!mul_ok(bh, (uint64_t)Tq, &rows)) return 0;
    int nsplit, chunk;
    attn::decode_plan((int)bh, Tq, Tk, &nsplit, &chunk);
    uint64_t parts, bytes;
    if (!mul_ok(rows, (uint64_t)nsplit, &parts)) return 0;
    if (!mul_ok(parts, (uint64_t)(D + 1) * 4, &bytes)) return 0;
    if (bytes > UINT64_MAX - 1024) return 0;
    return (size_t)((bytes + 256 + 255) & ~(uint64_t)255);
}

int attn_decode_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int B, int H, int Tq,
                       int Tk, int D, int causal, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o || !workspace) return ATTN_ERR_INVALID;
    if (B < 1 || H < 1 || Tq < 1 || Tk < 1 || D < 1) return ATTN_ERR_INVALID;
    if (Tq > Tk) return ATTN_ERR_INVALID;
    int st = check_shape(B, H, Tk, D, fwd16_head_dim(D));
    if (st != ATTN_OK) return st;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(workspace))
        return ATTN_ERR_INVALID;
    if (lse && !aligned4(lse)) return ATTN_ERR_INVALID;
    const size_t need = attn_decode_workspace_bytes(B, H, Tq, Tk, D);
    if (need == 0) return ATTN_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return ATTN_ERR_INVALID;
    if ((uint64_t)Tk * D * 2 > UINT32_MAX) return ATTN_ERR_UNSUPPORTED;
    int nsplit, chunk;
    const int BH = B * H;
    attn::decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    const uint64_t nqt = ((uint64_t)Tq + 31) / 32;
    if ((uint64_t)BH * nqt * nsplit > kMaxFusedWorkgroups ||
        ((uint64_t)BH * Tq + 3) / 4 > (uint64_t)INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    const double c = fabs((double)scale) * 1.4426950408889634073599;
    if (!isfinite((float)c)) return ATTN_ERR_INVALID;
    const uint64_t parts = (uint64_t)BH * Tq * nsplit;
    float* o_part = (float*)workspace;
    float* lse_part = o_part + parts * D;
    const hipError_t e = attn::launch_decode(q, k, v, o, lse, o_part, lse_part, BH, Tq, Tk, D,
                                             causal ? 1 : 0, (float)c, scale < 0.0f, dtype,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

static_assert(attn::kDecodeScratchBytes == ATTN_DECODE_SCRATCH_BYTES,
              "the header states the scratch size");

int attn_decode_noalloc_stream(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int H, int Tq, int Tk, int D, int causal,
                               float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
    if (B < 1 || H < 1 || Tq < 1 || Tk < 1 || D < 1) return ATTN_ERR_INVALID;
    if (Tq > Tk) return ATTN_ERR_INVALID;
    int st = check_shape(B, H, Tk, D, fwd16_head_dim(D));
    if (st != ATTN_OK) return st;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return ATTN_ERR_INVALID;
    if (lse && !aligned4(lse)) return ATTN_ERR_INVALID;
    if ((uint64_t)Tk * D * 2 > UINT32_MAX) return ATTN_ERR_UNSUPPORTED;
    uint64_t bh;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || bh > (uint64_t)INT32_MAX)
        return ATTN_ERR_UNSUPPORTED;
    const int BH = (int)bh;
    int nsplit, chunk;
    attn::decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    const uint64_t nqt = ((uint64_t)Tq + 31) / 32;
    if ((uint64_t)BH * nqt * nsplit > kMaxFusedWorkgroups) return ATTN_ERR_UNSUPPORTED;
    const size_t need = attn::decode_scratch_need(BH, Tq, Tk, D);
    if (need == 0 || need > attn::kDecodeScratchBytes) return ATTN_ERR_UNSUPPORTED;
    const double c = fabs((double)scale) * 1.4426950408889634073599;
    if (!isfinite((float)c)) return ATTN_ERR_INVALID;
    const hipError_t e = attn::launch_decode_noalloc(q, k, v, o, lse, BH, Tq, Tk, D,
                                                     causal ? 1 : 0, (float)c, scale < 0.0f,
                                                     dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

int attn_gated_recurrence_stream(const float* q, const float* k, const float* v,
                                 const float* gate, float* y, int B, int T, int H, int D,
                                 void* stream) {
    if (!q || !k || !v || !gate || !y) return ATTN_ERR_INVALID;
    if (B < 1 || T < 1 || H < 1 || D < 1) return ATTN_ERR_INVALID;
    if (!aligned4(q) || !aligned4(k) || !aligned4(v) || !aligned4(gate) || !aligned4(y))
        return ATTN_ERR_INVALID;
    if (D > kMaxRecurrenceDim) return ATTN_ERR_UNSUPPORTED;
    uint64_t bh, units, elems;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)(D + 7) / 8, &units) ||
        units > kMaxFusedWorkgroups)
        return ATTN_ERR_UNSUPPORTED;
    if (!mul_ok(bh * (uint64_t)D, (uint64_t)T, &elems) || elems > (uint64_t)INT64_MAX / 4)
        return ATTN_ERR_UNSUPPORTED;
    // one (batch, head) slice spans T steps of H * D floats, addressed with
    // 32-bit signed byte offsets
    if ((uint64_t)T * H * D * 4 > (uint64_t)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    const hipError_t e = attn::launch_recurrence(q, k, v, gate, y, B, T, H, D,
                                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

double attn_gated_recurrence_flops(int B, int T, int H, int D) {
    if (B < 1 || T < 1 || H < 1 || D < 1) return 0.0;
    return 5.0 * B * (double)T * H * (double)D * D;
}

double attn_bwd_flops(int B, int H, int T, int D, int causal) {
    return 2.5 * attn_flops(B, H, T, D, causal);
}

size_t attn_naive_workspace_bytes(int B, int H, int T) {
    if (B < 1 || H < 1 || T < 1) return 0;
    uint64_t bh, tt, table, two, rows, total;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &bh)) return 0;
    if (!mul_ok((uint64_t)T, (uint64_t)T, &tt)) return 0;
    if (!mul_ok(bh, tt, &table)) return 0;
    if (!mul_ok(table, 2, &two)) return 0;
    rows = bh * (uint64_t)T;
    if (two + rows < two) return 0;
    if (!mul_ok(two + rows, 4, &total)) return 0;
    if (total > UINT64_MAX - 255) return 0;
    return (size_t)((total + 255) & ~(uint64_t)255);
}

int attn_naive_fwd(const float* q, const float* k, const float* v, float* o,
                   float* lse, void* workspace, size_t workspace_bytes, int B,
                   int H, int T, int D, int causal, float scale, int dtype,
                   void* stream) {
    if (!q || !k || !v || !o || !workspace) return ATTN_ERR_INVALID;
    int st = check_shape(B, H, T, D, D == attn::kHeadDim);
    if (st != ATTN_OK) return st;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    if (dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(workspace))
        return ATTN_ERR_INVALID;
    if (lse && !aligned4(lse)) return ATTN_ERR_INVALID;
    const size_t need = attn_naive_workspace_bytes(B, H, T);
    if (need == 0) return ATTN_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return ATTN_ERR_INVALID;
    // grid limits of the three kernels: y and z dimensions stay <= 65535
    const uint64_t tiles = ((uint64_t)T + 63) / 64;
    if ((uint64_t)B * H > 65535 || tiles > 65535) return ATTN_ERR_UNSUPPORTED;
    const uint64_t table = (uint64_t)B * H * T * T;
    float* s = (float*)workspace;
    float* p = s + table;
    float* rowsum = p + table;
    const hipError_t e =
        attn::launch_naive(q, k, v, o, lse, s, p, rowsum, B * H, T,
                           causal ? 1 : 0, scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return ATTN_OK;
}

int attn_fused_tile(int dtype, int* block_m, int* block_n) {
    if (!valid_dtype(dtype) || !block_m || !block_n) return ATTN_ERR_INVALID;
    *block_m = attn::kBlockM;
    *block_n = dtype == ATTN_F32 ? attn::kBlockN32 : attn::kBlockN16;
    return ATTN_OK;
}

int attn_fused_kernel(int B, int H, int T, int D, int causal, int dtype) {
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    const int st = check_shape(B, H, T, D,
                               dtype == ATTN_F32 ? D == attn::kHeadDim : fwd16_head_dim(D));
    if (st != ATTN_OK) return st;
    // kernel table order (attn_kernel_name): fused 16-bit / fp32 first,
    // the head-dimension kernels after the decode ones, the eight-wave
    // kernels last; within each group bf16 before f16, causal before full
    const int full = causal ? 0 : 1, f16 = dtype == ATTN_F16 ? 2 : 0;
    const long long bh = (long long)B * H;
    if (dtype == ATTN_F32) return (attn::fwd32_split(bh, T) ? 6 : 4) + full;
    if (D != attn::kHeadDim) {
        const int hd0 = attn::kFusedKernels + attn::kNaiveKernels + attn::kBwdKernels +
                        attn::kDecodeKernels;
        return hd0 + (D == 128 ? 4 : 0) + f16 + full;
    }
    if (attn::fwd16_eight_waves(bh, T, causal != 0))
        return attn_kernel_count() - attn::kFwdW8Kernels + f16 + full;
    if (attn::fwd16_key_split(bh, T, causal != 0))
        return attn_kernel_count() - attn::kFwdW8Kernels + 4 + f16 + full;
    return f16 + full;
}

int attn_traffic_bytes(int path, int B, int H, int T, int D, int dtype,
                       int causal, attn_traffic* out) {
    if (!out) return ATTN_ERR_INVALID;
    if (!valid_dtype(dtype)) return ATTN_ERR_INVALID;
    const bool dim_ok = path == ATTN_PATH_FUSED && dtype != ATTN_F32 ? fwd16_head_dim(D)
                                                                     : D == attn::kHeadDim;
    int st = check_shape(B, H, T, D, dim_ok);
    if (st != ATTN_OK) return st;
    if (path != ATTN_PATH_FUSED && path != ATTN_PATH_NAIVE)
        return ATTN_ERR_INVALID;
    if (path == ATTN_PATH_NAIVE && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t elt = (uint64_t)elem_bytes(dtype);
    const uint64_t row_bytes = (uint64_t)D * elt;   // one row of q/k/v/o
    const uint64_t tensor = bh * (uint64_t)T * row_bytes;
    const uint64_t lse_bytes = bh * (uint64_t)T * 4;
    attn_traffic r;
    memset(&r, 0, sizeof(r));
    r.floor = 4 * tensor + lse_bytes;
    if (path == ATTN_PATH_FUSED) {
        // K and V rows each query tile loads (rows >= T are never fetched)
        int bm, bn;
        attn_fused_tile(dtype, &bm, &bn);
        // fp32 on a small grid runs the key-split kernel on 32-row tiles;
        // 16-bit D = 64 on a large one the eight-wave kernel on 256-row tiles
        if (dtype == ATTN_F32 && attn::fwd32_split((long long)bh, T)) bm = attn::kSplitRows;
        if (dtype != ATTN_F32 && D == attn::kHeadDim &&
            attn::fwd16_eight_waves((long long)bh, T, causal != 0))
            bm = attn::kBlockM8;
        const int nq = (T + bm - 1) / bm;
        uint64_t kv_rows = 0;
        for (int qt = 0; qt < nq; ++qt) {
            const int tiles = attn::key_tiles(qt, T, bn, causal != 0, bm);
            const uint64_t rows = (uint64_t)tiles * bn;
            kv_rows += rows < (uint64_t)T ? rows : (uint64_t)T;
        }
        r.ask = 2 * tensor + lse_bytes + 2 * bh * kv_rows * row_bytes;
    } else {
        const uint64_t tt = (uint64_t)T * T;
        r.score_matrix = 5 * 4 * bh * tt;
        r.table_bytes = attn_naive_workspace_bytes(B, H, T);
        // scores: each 64 x 64 tile reads a 64-row block of Q and of K;
        // weighted V: each 64-row block reads all of V; row sums written and
        // read once; O and lse written once.
        const uint64_t tiles = ((uint64_t)T + 63) / 64;
        r.ask = r.score_matrix + 2 * tensor * tiles + tensor * tiles +
                2 * lse_bytes + tensor + lse_bytes;
    }
    *out = r;
    return ATTN_OK;
}

double attn_flops(int B, int H, int T, int D, int causal) {
    if (B < 1 || H < 1 || T < 1 || D < 1) return 0.0;
    const double full = 4.0 * B * H * (double)T * (double)T * D;
    return causal ? full / 2.0 : full;
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported request";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_kernel_count(void) {
    return attn::kFusedKernels + attn::kNaiveKernels + attn::kBwdKernels +
           attn::kDecodeKernels + attn::kHdKernels + attn::kRecurrenceKernels +
           attn::kBwdAtomicKernels + attn::kDecodeHdKernels + attn::kDecodeMergedKernels +
           attn::kFwdW8Kernels;
}

const char* attn_kernel_name(int kernel) {
    static const char* const names[] = {
        "fused_fwd16<bf16, causal>", "fused_fwd16<bf16, full>",
        "fused_fwd16<f16, causal>",  "fused_fwd16<f16, full>",
        "fused_fwd32<causal>",       "fused_fwd32<full>",
        "fused_fwd32_split<causal>", "fused_fwd32_split<full>",
        "naive_scores",              "naive_softmax",
        "naive_weighted_v",
        "bwd_delta16<bf16>",         "bwd_kv16<bf16, causal>",
        "bwd_kv16<bf16, full>",      "bwd_q16<bf16, causal>",
        "bwd_q16<bf16, full>",       "bwd_delta16<f16>",
        "bwd_kv16<f16, causal>",     "bwd_kv16<f16, full>",
        "bwd_q16<f16, causal>",      "bwd_q16<f16, full>",
        "decode_split16<bf16, causal>", "decode_split16<bf16, full>",
        "decode_combine16<bf16>",    "decode_split16<f16, causal>",
        "decode_split16<f16, full>", "decode_combine16<f16>",
        "fused_hd16<bf16, causal, 32>", "fused_hd16<bf16, full, 32>",
        "fused_hd16<f16, causal, 32>", "fused_hd16<f16, full, 32>",
        "fused_hd16<bf16, causal, 128>", "fused_hd16<bf16, full, 128>",
        "fused_hd16<f16, causal, 128>", "fused_hd16<f16, full, 128>",
        "gated_recurrence32<D <= 8>",  "gated_recurrence32<D <= 16>",
        "gated_recurrence32<D <= 24>", "gated_recurrence32<D <= 32>",
        "gated_recurrence32<D <= 40>", "gated_recurrence32<D <= 48>",
        "gated_recurrence32<D <= 56>", "gated_recurrence32<D <= 64>",
        "gated_recurrence_wave32<D <= 8>",  "gated_recurrence_wave32<D <= 16>",
        "gated_recurrence_wave32<D <= 24>", "gated_recurrence_wave32<D <= 32>",
        "gated_recurrence_wave32<D <= 40>", "gated_recurrence_wave32<D <= 48>",
        "gated_recurrence_wave32<D <= 56>", "gated_recurrence_wave32<D <= 64>",
        "bwd_prep16<bf16>",          "bwd_kvq16<bf16, causal>",
        "bwd_kvq16<bf16, full>",     "bwd_dq_finish16<bf16>",
        "bwd_prep16<f16>",           "bwd_kvq16<f16, causal>",
        "bwd_kvq16<f16, full>",      "bwd_dq_finish16<f16>",
        "decode_split16<bf16, causal, 32>", "decode_split16<bf16, full, 32>",
        "decode_combine16<bf16, 32>", "decode_split16<f16, causal, 32>",
        "decode_split16<f16, full, 32>", "decode_combine16<f16, 32>",
        "decode_split16<bf16, causal, 128>", "decode_split16<bf16, full, 128>",
        "decode_combine16<bf16, 128>", "decode_split16<f16, causal, 128>",
        "decode_split16<f16, full, 128>", "decode_combine16<f16, 128>",
        "decode_merged16<bf16, causal>", "decode_merged16<bf16, full>",
        "decode_merged16<f16, causal>", "decode_merged16<f16, full>",
        "decode_merged16<bf16, causal, 32>", "decode_merged16<bf16, full, 32>",
        "decode_merged16<f16, causal, 32>", "decode_merged16<f16, full, 32>",
        "decode_merged16<bf16, causal, 128>", "decode_merged16<bf16, full, 128>",
        "decode_merged16<f16, causal, 128>", "decode_merged16<f16, full, 128>",
        "fused_fwd16w8<bf16, causal>", "fused_fwd16w8<bf16, full>",
        "fused_fwd16w8<f16, causal>",  "fused_fwd16w8<f16, full>",
        "fused_fwd16w8s<bf16, causal>", "fused_fwd16w8s<bf16, full>",
        "fused_fwd16w8s<f16, causal>",  "fused_fwd16w8s<f16, full>"};
    if (kernel < 0 || kernel >= attn_kernel_count()) return nullptr;
    return names[kernel];
}

int attn_kernel_attributes(int kernel, attn_kernel_attr* out) {
    if (!out || kernel < 0 || kernel >= attn_kernel_count())
        return ATTN_ERR_INVALID;
    const int naive0 = attn::kFusedKernels, bwd0 = naive0 + attn::kNaiveKernels;
    const int dec0 = bwd0 + attn::kBwdKernels, hd0 = dec0 + attn::kDecodeKernels;
    const int rec0 = hd0 + attn::kHdKernels;
    const int bat0 = rec0 + attn::kRecurrenceKernels;
    const int dhd0 = bat0 + attn::kBwdAtomicKernels;
    const int dmg0 = dhd0 + attn::kDecodeHdKernels;
    const int w80 = dmg0 + attn::kDecodeMergedKernels;
    const void* fn = kernel >= w80    ? attn::fused_w8_kernel_ptr(kernel - w80)
                     : kernel < naive0  ? attn::fused_kernel_ptr(kernel)
                     : kernel < bwd0 ? attn::naive_kernel_ptr(kernel - naive0)
                     : kernel < dec0 ? attn::bwd_kernel_ptr(kernel - bwd0)
                     : kernel < hd0  ? attn::decode_kernel_ptr(kernel - dec0)
                     : kernel < rec0 ? attn::hd_kernel_ptr(kernel - hd0)
                     : kernel < bat0 ? attn::recurrence_kernel_ptr(kernel - rec0)
                     : kernel < dhd0 ? attn::bwd_atomic_kernel_ptr(kernel - bat0)
                     : kernel < dmg0 ? attn::decode_kernel_ptr(6 + kernel - dhd0)
                                     : attn::decode_merged_kernel_ptr(kernel - dmg0);
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return hip_fail(e);
    // threads per workgroup of the kernel's launches: the recurrence's
    // kernel i runs i + 1 waves
    const int threads = kernel >= w80 ? attn::kThreads8
                        : kernel >= 6 && kernel < naive0 ? attn::kSplitThreads
                        : kernel >= bat0     ? attn::kThreads
                        : kernel >= rec0 + 8 ? 64
                        : kernel >= rec0   ? 64 * (kernel - rec0 + 1)
                                           : attn::kThreads;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0);
    if (e != hipSuccess) return hip_fail(e);
    out->num_regs = fa.numRegs;
    out->lds_bytes = (int)fa.sharedSizeBytes;
    out->private_bytes = (int)fa.localSizeBytes;
    out->threads_per_workgroup = threads;
    out->workgroups_per_cu = per_cu;
    return ATTN_OK;
}

}  // extern "C"
