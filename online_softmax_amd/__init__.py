"""MI355X-native exact attention on gfx950: the fused online-softmax forward
(head dims 32, 64, 128), its backward pass, decode against a key/value
cache, and the gated linear recurrence.

The kernels and the materialising contrast path live in libattn.so (csrc/,
C ABI in include/attn.h); this package is its thin binding. Nothing here computes attention: every step runs in the HIP kernels,
and without the built library every call raises.
"""
from .binding import (  # noqa: F401
    ATTN_BF16, ATTN_ERR_HIP, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_F16,
    ATTN_F32, ATTN_OK, ATTN_PATH_FUSED, ATTN_PATH_NAIVE, EXPORTS, LIBRARY,
    AttnError, attention, attention_backward, attention_decode, attn_bwd_flops,
    attn_bwd_stream, attn_bwd_atomic_stream, attn_bwd_atomic_workspace_bytes,
    attn_decode_stream, attn_decode_workspace_bytes, attn_decode_noalloc_stream,
    attn_bwd_workspace_bytes, attn_flops, attn_fused_tile, attn_fused_kernel, attn_fwd,
    attn_fwd_stream, attn_kernel_attributes, attn_kernel_count,
    attn_kernel_name, attn_last_hip_error, attn_naive_fwd,
    attn_naive_workspace_bytes, attn_status_string, attn_traffic_bytes,
    dtype_code, load, attn_gated_recurrence_stream, attn_gated_recurrence_flops,
    flash_attention, gated_recurrence)
