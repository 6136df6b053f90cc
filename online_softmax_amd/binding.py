"""ctypes binding of libattn.so (include/attn.h), argument marshalling only.

Every function here has the name of the C entry point it calls and takes
torch tensors where the C function takes device pointers; it derives the
sizes and the dtype code from the tensors, passes the current HIP stream
unless one is given, and raises AttnError for a non-OK status. No step of
the computation happens here, and there is no fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, -1, -2, -3
ATTN_PATH_FUSED, ATTN_PATH_NAIVE = 0, 1

# every symbol include/attn.h declares
EXPORTS = ("attn_fwd", "attn_fwd_stream", "attn_naive_fwd",
           "attn_naive_workspace_bytes", "attn_bwd_stream",
           "attn_bwd_workspace_bytes", "attn_bwd_atomic_stream",
           "attn_bwd_atomic_workspace_bytes", "attn_bwd_flops", "attn_decode_stream",
           "attn_decode_workspace_bytes", "attn_traffic_bytes",
           "attn_flops", "attn_status_string", "attn_last_hip_error",
           "attn_kernel_count", "attn_kernel_name", "attn_kernel_attributes",
           "attn_fused_tile", "attn_gated_recurrence_stream",
           "attn_gated_recurrence_flops", "attn_decode_noalloc_stream",
           "attn_fused_kernel")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib().attn_status_string(status).decode()
        hip = _lib().attn_last_hip_error() if status == ATTN_ERR_HIP else 0
        super().__init__(f"{where}: {text} ({status})" +
                         (f", hipError {hip}" if hip else ""))


class attn_traffic(ctypes.Structure):
    _fields_ = [("floor", ctypes.c_uint64), ("ask", ctypes.c_uint64),
                ("score_matrix", ctypes.c_uint64),
                ("table_bytes", ctypes.c_uint64)]


class attn_kernel_attr(ctypes.Structure):
    _fields_ = [("num_regs", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("private_bytes", ctypes.c_int),
                ("threads_per_workgroup", ctypes.c_int),
                ("workgroups_per_cu", ctypes.c_int)]


_lock = threading.Lock()
_handle = None


def load(path: str = LIBRARY):
    """Load the in-tree libattn.so; raises if it has not been built."""
    global _handle
    with _lock:
        if _handle is not None and path == LIBRARY:
            return _handle
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m online_softmax_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(path)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd_stream.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
        lib.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I]
        lib.attn_naive_fwd.argtypes = [P, P, P, P, P, P, S, I, I, I, I, I, F,
                                       I, P]
        lib.attn_naive_workspace_bytes.argtypes = [I, I, I]
        lib.attn_naive_workspace_bytes.restype = S
        lib.attn_bwd_stream.argtypes = [P] * 10 + [S, I, I, I, I, I, F, I, P]
        lib.attn_bwd_workspace_bytes.argtypes = [I, I, I]
        lib.attn_bwd_workspace_bytes.restype = S
        lib.attn_bwd_atomic_stream.argtypes = [P] * 10 + [S, I, I, I, I, I, F, I, P]
        lib.attn_bwd_atomic_workspace_bytes.argtypes = [I, I, I]
        lib.attn_bwd_atomic_workspace_bytes.restype = S
        lib.attn_bwd_flops.argtypes = [I, I, I, I, I]
        lib.attn_bwd_flops.restype = ctypes.c_double
        lib.attn_decode_stream.argtypes = [P] * 6 + [S, I, I, I, I, I, I, F, I, P]
        lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.attn_decode_workspace_bytes.restype = S
        lib.attn_decode_noalloc_stream.argtypes = [P] * 5 + [I, I, I, I, I, I, F, I, P]
        lib.attn_gated_recurrence_stream.argtypes = [P] * 5 + [I, I, I, I, P]
        lib.attn_gated_recurrence_flops.argtypes = [I, I, I, I]
        lib.attn_gated_recurrence_flops.restype = ctypes.c_double
        lib.attn_traffic_bytes.argtypes = [I, I, I, I, I, I, I,
                                           ctypes.POINTER(attn_traffic)]
        lib.attn_flops.argtypes = [I, I, I, I, I]
        lib.attn_flops.restype = ctypes.c_double
        lib.attn_status_string.argtypes = [I]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_hip_error.argtypes = []
        lib.attn_kernel_count.argtypes = []
        lib.attn_kernel_name.argtypes = [I]
        lib.attn_kernel_name.restype = ctypes.c_char_p
        lib.attn_kernel_attributes.argtypes = [I, ctypes.POINTER(attn_kernel_attr)]
        lib.attn_fused_tile.argtypes = [I, ctypes.POINTER(I), ctypes.POINTER(I)]
        lib.attn_fused_kernel.argtypes = [I, I, I, I, I, I]
        for name in EXPORTS:  # fail here, not at first use, if one is absent
            getattr(lib, name)
        if path == LIBRARY:
            _handle = lib
        return lib


def _lib():
    return load()


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def dtype_code(t) -> int:
    import torch
    codes = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16,
             torch.float16: ATTN_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name: str, shape, dtype, device):
    """Raise ValueError unless tensor t (None allowed only where the caller
    skips the check) is contiguous, on `device`, of `dtype` and `shape`: the
    C ABI takes bare pointers and trusts their extents."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(int(x) for x in t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_lse(lse, shape, device):
    import torch
    if lse is not None:
        _expect(lse, "lse", shape, torch.float32, device)


def _expect_workspace(ws, device):
    if ws is None or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream)) if stream else None


def _dims(q):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, D]")
    return tuple(int(x) for x in q.shape)


def attn_fwd_stream(q, k, v, o, lse, causal: bool, scale: float, stream=None):
    """Fused forward into caller-owned o ([B,H,T,D], q's dtype) and lse
    ([B,H,T] float32 or None) on `stream` (default: the current stream)."""
    B, H, T, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, name, q.shape, q.dtype, q.device)
    _expect_lse(lse, (B, H, T), q.device)
    st = _lib().attn_fwd_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                B, H, T, D, int(bool(causal)), float(scale),
                                dtype_code(q), _stream(stream, q.device))
    _check(st, "attn_fwd_stream")


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float):
    """Fused forward on the null stream."""
    B, H, T, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, name, q.shape, q.dtype, q.device)
    _expect_lse(lse, (B, H, T), q.device)
    st = _lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                         T, D, int(bool(causal)), float(scale), dtype_code(q))
    _check(st, "attn_fwd")


def attn_naive_workspace_bytes(B: int, H: int, T: int) -> int:
    return int(_lib().attn_naive_workspace_bytes(B, H, T))


def attn_naive_fwd(q, k, v, o, lse, workspace, causal: bool, scale: float,
                   stream=None):
    """Materialising fp32 path; workspace is a caller-owned device tensor of
    at least attn_naive_workspace_bytes(B, H, T) bytes."""
    B, H, T, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, name, q.shape, q.dtype, q.device)
    _expect_lse(lse, (B, H, T), q.device)
    _expect_workspace(workspace, q.device)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib().attn_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               _ptr(workspace), nbytes, B, H, T, D,
                               int(bool(causal)), float(scale), dtype_code(q),
                               _stream(stream, q.device))
    _check(st, "attn_naive_fwd")


def attn_bwd_workspace_bytes(B: int, H: int, T: int) -> int:
    return int(_lib().attn_bwd_workspace_bytes(B, H, T))


def _bwd_call(entry: str, q, k, v, o, dout, lse, dq, dk, dv, workspace, causal,
              scale, stream):
    B, H, T, D = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _expect(t, name, q.shape, q.dtype, q.device)
    import torch
    _expect(lse, "lse", (B, H, T), torch.float32, q.device)
    _expect_workspace(workspace, q.device)
    nbytes = workspace.numel() * workspace.element_size()
    st = getattr(_lib(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(workspace), nbytes, B, H, T, D,
                                int(bool(causal)), float(scale), dtype_code(q),
                                _stream(stream, q.device))
    _check(st, entry)


def attn_bwd_stream(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool,
                    scale: float, stream=None):
    """Backward pass into caller-owned dq, dk, dv (q's shape and dtype);
    workspace is a device tensor of at least attn_bwd_workspace_bytes(B, H,
    T) bytes."""
    _bwd_call("attn_bwd_stream", q, k, v, o, dout, lse, dq, dk, dv, workspace,
              causal, scale, stream)


def attn_bwd_atomic_workspace_bytes(B: int, H: int, T: int) -> int:
    return int(_lib().attn_bwd_atomic_workspace_bytes(B, H, T))


def attn_bwd_atomic_stream(q, k, v, o, dout, lse, dq, dk, dv, workspace,
                           causal: bool, scale: float, stream=None):
    """The backward pass with dQ summed by float32 atomics (one main kernel);
    workspace is a device tensor of at least
    attn_bwd_atomic_workspace_bytes(B, H, T) bytes."""
    _bwd_call("attn_bwd_atomic_stream", q, k, v, o, dout, lse, dq, dk, dv,
              workspace, causal, scale, stream)


def attn_decode_workspace_bytes(B: int, H: int, Tq: int, Tk: int, D: int = 64) -> int:
    return int(_lib().attn_decode_workspace_bytes(B, H, Tq, Tk, D))


def attn_decode_stream(q, k, v, o, lse, workspace, causal: bool, scale: float,
                       stream=None):
    """Decode: q [B, H, Tq, D] against the cache k, v [B, H, Tk, D] into o
    (q's shape) and lse ([B, H, Tq] float32 or None)."""
    B, H, Tq, D = _dims(q)
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Tk, D]")
    Tk = int(k.shape[2])
    _expect(q, "q", q.shape, q.dtype, q.device)
    _expect(o, "o", q.shape, q.dtype, q.device)
    for name, t in (("k", k), ("v", v)):
        _expect(t, name, (B, H, Tk, D), q.dtype, q.device)
    _expect_lse(lse, (B, H, Tq), q.device)
    _expect_workspace(workspace, q.device)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib().attn_decode_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(workspace), nbytes, B, H, Tq, Tk, D,
                                   int(bool(causal)), float(scale), dtype_code(q),
                                   _stream(stream, q.device))
    _check(st, "attn_decode_stream")


def attn_decode_noalloc_stream(q, k, v, o, lse, causal: bool, scale: float, stream=None):
    """Decode as attn_decode_stream, with the library's own scratch instead
    of a workspace (no allocation; calls on one GPU must not overlap)."""
    B, H, Tq, D = _dims(q)
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Tk, D]")
    Tk = int(k.shape[2])
    _expect(q, "q", q.shape, q.dtype, q.device)
    _expect(o, "o", q.shape, q.dtype, q.device)
    for name, t in (("k", k), ("v", v)):
        _expect(t, name, (B, H, Tk, D), q.dtype, q.device)
    _expect_lse(lse, (B, H, Tq), q.device)
    st = _lib().attn_decode_noalloc_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                           B, H, Tq, Tk, D, int(bool(causal)), float(scale),
                                           dtype_code(q), _stream(stream, q.device))
    _check(st, "attn_decode_noalloc_stream")


def attn_gated_recurrence_stream(q, k, v, gate, y, stream=None):
    """Gated linear recurrence into caller-owned y; q, k, v, gate and y are
    float32 [B, T, H, D] device tensors."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, D]")
    B, T, H, D = (int(x) for x in q.shape)
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("y", y)):
        _expect(t, name, q.shape, torch.float32, q.device)
    st = _lib().attn_gated_recurrence_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(y),
                                             B, T, H, D, _stream(stream, q.device))
    _check(st, "attn_gated_recurrence_stream")


def gated_recurrence(q, k, v, gate, stream=None):
    """Allocate y with torch on q's device and run the gated recurrence."""
    import torch
    y = torch.empty_like(q)
    attn_gated_recurrence_stream(q, k, v, gate, y, stream)
    return y


def attn_gated_recurrence_flops(B: int, T: int, H: int, D: int) -> float:
    return float(_lib().attn_gated_recurrence_flops(B, T, H, D))


def attn_bwd_flops(B: int, H: int, T: int, D: int, causal: bool) -> float:
    return float(_lib().attn_bwd_flops(B, H, T, D, int(bool(causal))))


def attn_traffic_bytes(path: int, B: int, H: int, T: int, D: int, dtype: int,
                       causal: bool) -> dict:
    out = attn_traffic()
    st = _lib().attn_traffic_bytes(path, B, H, T, D, dtype, int(bool(causal)),
                                   ctypes.byref(out))
    _check(st, "attn_traffic_bytes")
    return {f: int(getattr(out, f)) for f, _ in attn_traffic._fields_}


def attn_flops(B: int, H: int, T: int, D: int, causal: bool) -> float:
    return float(_lib().attn_flops(B, H, T, D, int(bool(causal))))


def attn_fused_tile(dtype: int):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(_lib().attn_fused_tile(dtype, ctypes.byref(bm), ctypes.byref(bn)),
           "attn_fused_tile")
    return bm.value, bn.value


def attn_fused_kernel(B: int, H: int, T: int, D: int, causal: bool, dtype: int) -> int:
    """Kernel-table index of the kernel attn_fwd launches for these
    arguments (see attn_kernel_name)."""
    r = int(_lib().attn_fused_kernel(B, H, T, D, int(bool(causal)), dtype))
    _check(r if r < 0 else ATTN_OK, "attn_fused_kernel")
    return r


def attn_status_string(status: int) -> str:
    return _lib().attn_status_string(status).decode()


def attn_last_hip_error() -> int:
    return int(_lib().attn_last_hip_error())


def attn_kernel_count() -> int:
    return int(_lib().attn_kernel_count())


def attn_kernel_name(kernel: int) -> str:
    r = _lib().attn_kernel_name(kernel)
    return None if r is None else r.decode()


def attn_kernel_attributes(kernel: int) -> dict:
    out = attn_kernel_attr()
    _check(_lib().attn_kernel_attributes(kernel, ctypes.byref(out)),
           "attn_kernel_attributes")
    return {f: int(getattr(out, f)) for f, _ in attn_kernel_attr._fields_}


def attention(q, k, v, causal: bool = True, scale: float | None = None,
              with_lse: bool = True, stream=None):
    """Allocate o (and lse) with torch on q's device and run the fused path.
    Returns (o, lse)."""
    import torch
    B, H, T, D = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) \
        if with_lse else None
    attn_fwd_stream(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = True,
                       scale: float | None = None, stream=None,
                       atomic: bool = False):
    """Allocate dq, dk, dv and the workspace with torch on q's device and run
    the backward pass for the forward (o, lse) of the same q, k, v, causal and
    scale: the two-kernel split, or with atomic=True the single main kernel
    that sums dQ with atomics. Returns (dq, dk, dv)."""
    import torch
    B, H, T, D = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = (attn_bwd_atomic_workspace_bytes if atomic else attn_bwd_workspace_bytes)(B, H, T)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    run = attn_bwd_atomic_stream if atomic else attn_bwd_stream
    run(q, k, v, o, dout, lse, dq, dk, dv, ws, causal, scale, stream)
    return dq, dk, dv


_FLASH_FN = None


def _flash_function():
    """The autograd Function pairing attn_fwd_stream with the backward entry
    points, made once (torch is imported lazily, as everywhere here)."""
    global _FLASH_FN
    if _FLASH_FN is not None:
        return _FLASH_FN
    import torch

    class FlashAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, atomic):
            q, k, v = (x.contiguous() for x in (q, k, v))
            o, lse = attention(q, k, v, causal, scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale, ctx.atomic = causal, scale, atomic
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            if q.dtype not in (torch.bfloat16, torch.float16):
                raise AttnError(ATTN_ERR_UNSUPPORTED,
                                "flash_attention backward: the backward pass takes bf16 or f16 "
                                f"inputs, not {q.dtype}")
            dq, dk, dv = attention_backward(q, k, v, o, lse, dout.contiguous(), ctx.causal,
                                            ctx.scale, atomic=ctx.atomic)
            return dq, dk, dv, None, None, None

    _FLASH_FN = FlashAttention
    return _FLASH_FN


def flash_attention(q, k, v, causal: bool = True, scale: float | None = None,
                    atomic: bool = False):
    """O = softmax(Q K^T * scale + causal mask) V for q, k, v [B, H, T, D] as
    a torch autograd function: the user-facing call of "Flash attention in
    PyTorch, then in Triton" (section "Backwards, and training with it"),
    whose forward saves q, k, v, O and the log-sum-exps and whose backward
    recomputes the probabilities from them. Both passes run this library's
    kernels (the backward: the two-kernel split, or with atomic=True the
    single kernel summing dQ with atomics). Under autocast q, k and v are
    first cast to autocast's dtype, as that page's function does (rotary
    embeddings leave q and k in float32 while v is bf16). Inputs are made
    contiguous. scale defaults to 1/sqrt(D)."""
    import torch
    if torch.is_autocast_enabled(q.device.type):
        dt = torch.get_autocast_dtype(q.device.type)
        q, k, v = (x.to(dt) for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(int(q.shape[-1]))
    return _flash_function().apply(q, k, v, bool(causal), float(scale), bool(atomic))


def attention_decode(q, k, v, causal: bool = True, scale: float | None = None,
                     stream=None):
    """Allocate o, lse and the workspace with torch and run the decode path.
    Returns (o, lse)."""
    import torch
    B, H, Tq, D = _dims(q)
    Tk = int(k.shape[2])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    ws = torch.empty(attn_decode_workspace_bytes(B, H, Tq, Tk, D), dtype=torch.uint8,
                     device=q.device)
    attn_decode_stream(q, k, v, o, lse, ws, causal, scale, stream)
    return o, lse
