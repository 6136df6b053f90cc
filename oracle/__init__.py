"""Double-precision CPU attention oracle (ctypes binding of attn_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The GPU library never imports, links
or executes anything in this directory, and this directory never imports the
GPU library.

The oracle evaluates exact attention row by row in double precision with the
row maximum subtracted before the exponential, as the double-precision CPU
reference of the page "attention.cu" does, with the causal mask and the
log-sum-exp output of "Flash attention in PyTorch, then in Triton" (sections
"Attention by hand" and "Backwards, and training with it"). The log-sum-exp
is returned in natural-log units.

Parity pins live in tests/test_oracle_pins.py; every function here has one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
# The mutation test of the pins points this at deliberately broken builds of
# a copy of the source; everything else uses the in-tree library.
LIBRARY = os.environ.get("ATTN_ORACLE_LIBRARY",
                         os.path.join(_HERE, "liboracle.so"))

# -O2, no fast-math, no floating-point contraction: every product and sum is
# a separately rounded double operation.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
          "-ffp-contract=off", "-fno-fast-math"]

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc; returns the path."""
    if not force and os.path.exists(LIBRARY) and \
            os.path.getmtime(LIBRARY) >= os.path.getmtime(SOURCE):
        return LIBRARY
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                build()
            lib = ctypes.CDLL(LIBRARY)
            f = lib.oracle_attention
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 4 + [
                ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int]
            g = lib.oracle_probabilities
            g.restype = ctypes.c_int
            g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                          ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                          ctypes.c_void_p]
            d = lib.oracle_attention_kv
            d.restype = ctypes.c_int
            d.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5 + [
                ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int]
            r = lib.oracle_gated_recurrence
            r.restype = ctypes.c_int
            r.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [
                ctypes.c_void_p, ctypes.c_int]
            b = lib.oracle_attention_backward
            b.restype = ctypes.c_int
            b.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [
                ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                ctypes.c_int64] + [ctypes.c_void_p] * 3 + [ctypes.c_int]
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle uses by default on this host."""
    return int(_load().oracle_max_threads())


def _as_f32(x) -> np.ndarray:
    """Widen to a C-contiguous float32 numpy array (exact for bf16/fp16)."""
    try:  # torch tensors are accepted too (CPU, any float dtype)
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if x.dtype != np.float32:
        x = x.astype(np.float32)
    return np.ascontiguousarray(x)


def attention(q, k, v, causal: bool, scale: float, rows=None,
              threads: int = 0):
    """Exact attention in double precision.

    q, k, v: [B, H, T, D] (or [T, D] for one head), float32 or exactly
    widenable to it. rows: optional 1-D int array of flat row ids
    (b * H + h) * T + t. Returns (o, lse) as float64: o is [B, H, T, D]
    (or [len(rows), D]), lse is [B, H, T] (or [len(rows)]).
    """
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    single = q.ndim == 2
    if single:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, T, D] shape")
    B, H, T, D = q.shape
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
        o = np.empty((n, D), np.float64)
        lse = np.empty((n,), np.float64)
        rptr = rows.ctypes.data
    else:
        n = B * H * T
        o = np.empty((B, H, T, D), np.float64)
        lse = np.empty((B, H, T), np.float64)
        rptr = None
    rc = _load().oracle_attention(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, T, D,
        int(bool(causal)), float(scale), rptr, n, o.ctypes.data,
        lse.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle_attention failed (%d)" % rc)
    if single and rows is None:
        return o[0, 0], lse[0, 0]
    return o, lse


def probabilities(q, k, causal: bool, scale: float) -> np.ndarray:
    """Full [T, T] softmax-weight table of one head (q, k: [T, D])."""
    q, k = _as_f32(q), _as_f32(k)
    if q.ndim != 2 or q.shape != k.shape:
        raise ValueError("q, k must share one [T, D] shape")
    T, D = q.shape
    P = np.empty((T, T), np.float64)
    rc = _load().oracle_probabilities(q.ctypes.data, k.ctypes.data, T, D,
                                      int(bool(causal)), float(scale),
                                      P.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_probabilities failed (%d)" % rc)
    return P


def attention_backward(q, k, v, dout, causal: bool, scale: float,
                       slices=None, threads: int = 0):
    """Exact gradients of attention in double precision.

    q, k, v, dout: [B, H, T, D] (or [T, D] for one head), float32 or exactly
    widenable to it; dout is the gradient of the loss with respect to the
    output. slices: optional 1-D int array of slice ids b * H + h. Returns
    (dq, dk, dv) as float64, each [B, H, T, D] (or [len(slices), T, D], or
    [T, D] for one head), following "Flash attention in PyTorch, then in
    Triton", section "Backwards, and training with it".
    """
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    single = q.ndim == 2
    if single:
        q, k, v, dout = q[None, None], k[None, None], v[None, None], dout[None, None]
    if q.ndim != 4 or any(x.shape != q.shape for x in (k, v, dout)):
        raise ValueError("q, k, v, dout must share one [B, H, T, D] shape")
    B, H, T, D = q.shape
    if slices is not None:
        slices = np.ascontiguousarray(np.asarray(slices, dtype=np.int64))
        n = slices.shape[0]
        shape = (n, T, D)
        sptr = slices.ctypes.data
    else:
        n = B * H
        shape = (B, H, T, D)
        sptr = None
    dq = np.empty(shape, np.float64)
    dk = np.empty(shape, np.float64)
    dv = np.empty(shape, np.float64)
    rc = _load().oracle_attention_backward(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, H,
        T, D, int(bool(causal)), float(scale), sptr, n, dq.ctypes.data,
        dk.ctypes.data, dv.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle_attention_backward failed (%d)" % rc)
    if single and slices is None:
        return dq[0, 0], dk[0, 0], dv[0, 0]
    return dq, dk, dv


def attention_kv(q, k, v, causal: bool, scale: float, threads: int = 0):
    """Exact attention of Tq new queries against a Tk-token key/value cache
    (decode), in double precision: q [B, H, Tq, D], k and v [B, H, Tk, D],
    Tq <= Tk; query i sits at position Tk - Tq + i, so the causal mask is
    aligned to the bottom-right of the table. Returns (o [B, H, Tq, D],
    lse [B, H, Tq]) as float64."""
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q [B, H, Tq, D] and k, v [B, H, Tk, D] expected")
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    o = np.empty((B, H, Tq, D), np.float64)
    lse = np.empty((B, H, Tq), np.float64)
    rc = _load().oracle_attention_kv(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                     B, H, Tq, Tk, D, int(bool(causal)),
                                     float(scale), o.ctypes.data,
                                     lse.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle_attention_kv failed (%d)" % rc)
    return o, lse


def gated_recurrence(q, k, v, gate, threads: int = 0):
    """The gated linear recurrence of the page "Kimi-K2.6 l2 p24"
    (POPCORNBENCH) in double precision: per (batch, head) a D x D state S
    from zero; at each step t, S[i, j] = gate[t, j] S[i, j] + k[t, i] v[t, j],
    then y[t, j] = sum_i q[t, i] S[i, j]. q, k, v, gate: [B, T, H, D] float32
    (or exactly widenable); returns y [B, T, H, D] float64."""
    q, k, v, gate = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(gate)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape == gate.shape):
        raise ValueError("q, k, v, gate must share one [B, T, H, D] shape")
    B, T, H, D = q.shape
    y = np.empty((B, T, H, D), np.float64)
    rc = _load().oracle_gated_recurrence(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         gate.ctypes.data, B, T, H, D, y.ctypes.data,
                                         int(threads))
    if rc != 0:
        raise RuntimeError("oracle_gated_recurrence failed (%d)" % rc)
    return y
