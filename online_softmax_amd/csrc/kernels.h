// Internal launchers shared by the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// element type codes (match attn_dtype in include/attn.h)
#define ATTN_DT_F32 0
#define ATTN_DT_BF16 1
#define ATTN_DT_F16 2

namespace attn {

// Fused online-softmax forward over BH = B*H slices of T rows each.
// c = |scale| * log2(e); negate_q flips the sign of Q (for scale < 0).
hipError_t launch_fused(const void* q, const void* k, const void* v, void* o,
                        float* lse, int BH, int T, int causal, float c,
                        bool negate_q, int dt, hipStream_t stream);

// Materialising fp32 path. s, p: [BH, T, T]; rowsum: [BH, T].
hipError_t launch_naive(const float* q, const float* k, const float* v,
                        float* o, float* lse, float* s, float* p,
                        float* rowsum, int BH, int T, int causal, float scale,
                        hipStream_t stream);

// Backward pass (16-bit dtypes): delta = rowsum(dO * O) into the row
// workspace `ws` (bwd_ws_stride in fused_layout.h: -delta, then lse *
// log2(e), float32 per row), then dK/dV and dQ. c = |scale| * log2(e);
// negate flips the sign of the scores (for scale < 0); scale multiplies dQ
// and dK.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* ws, int BH, int T, int causal, float c, float scale,
                      bool negate, int dt, hipStream_t stream);

// Backward pass in one main kernel (16-bit dtypes): delta into `delta` and
// zeros into `dq_acc` ([BH, T, 64] float32), then dK/dV with the dQ sums
// added to dq_acc by atomics, then dq = scale * dq_acc.
hipError_t launch_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, float* dq_acc, int BH, int T, int causal, float c,
                             float scale, bool negate, int dt, hipStream_t stream);

// Decode: Tq queries against a Tk-token cache (head dimension D = 32, 64 or
// 128), split over the keys into o_part [BH*Tq, nsplit, D] and lse_part
// [BH*Tq, nsplit] (float32), then merged; the split is decode_plan
// (fused_layout.h).
hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                         float* o_part, float* lse_part, int BH, int Tq, int Tk, int D,
                         int causal, float c, bool negate_q, int dt, hipStream_t stream);

// Decode without allocation: the same split, with the partials in the
// library's static scratch and the merge done by the last workgroup of each
// query tile (one launch). The scratch holds kDecodeCounters tile counters
// and up to kDecodePartRows (row, split) partials of D <= 128.
constexpr int kDecodeCounters = 256;
constexpr size_t kDecodeCounterBytes = 1024;
constexpr size_t kDecodePartRows = 8192;
constexpr size_t kDecodeScratchBytes = kDecodeCounterBytes + kDecodePartRows * (128 + 1) * 4;
// Scratch bytes a call needs (0: the sizes do not fit its tile counters).
size_t decode_scratch_need(int BH, int Tq, int Tk, int D);
hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int BH, int Tq, int Tk, int D, int causal,
                                 float c, bool negate_q, int dt, hipStream_t stream);

// Fused forward for head dimensions 32 and 128 (16-bit dtypes only).
hipError_t launch_fused_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int BH, int T, int D, int causal, float c, bool negate_q, int dt,
                           hipStream_t stream);

// Gated linear recurrence (float32, [B, T, H, D], D <= 64).
hipError_t launch_recurrence(const float* q, const float* k, const float* v, const float* gate,
                             float* y, int B, int T, int H, int D, hipStream_t stream);

// Kernel table for attribute queries.
constexpr int kFusedKernels = 8;
constexpr int kNaiveKernels = 3;
constexpr int kBwdKernels = 10;
constexpr int kDecodeKernels = 6;
constexpr int kHdKernels = 8;
constexpr int kRecurrenceKernels = 16;
constexpr int kBwdAtomicKernels = 8;
constexpr int kDecodeHdKernels = 12;  // decode at D = 32 and 128 (decode_kernel_ptr 6 .. 17)
constexpr int kDecodeMergedKernels = 12;  // decode without allocation, D = 64, 32, 128
constexpr int kFwdW8Kernels = 8;          // 8-wave 16-bit forward and its key split, D = 64
const void* fused_kernel_ptr(int index);
const void* naive_kernel_ptr(int index);
const void* bwd_kernel_ptr(int index);
const void* decode_kernel_ptr(int index);  // 0 .. 5 at D = 64, then D = 32, 128
const void* hd_kernel_ptr(int index);
const void* recurrence_kernel_ptr(int index);
const void* bwd_atomic_kernel_ptr(int index);
const void* decode_merged_kernel_ptr(int index);
const void* fused_w8_kernel_ptr(int index);

}  // namespace attn
