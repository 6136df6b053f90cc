"""GPU parity of the single-kernel backward (dQ summed by float32 atomics):
dQ, dK, dV through attn_bwd_atomic_stream against the double oracle's
gradients of the same seeded 16-bit inputs, with the bound of the split
backward's tests (2e-2 times max(1, max |g|) per gradient tensor; the
products round P and dS to the 16-bit type as there, and the float32 sum of
dQ only changes its order).
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_qkv
from conftest import flush_print
from test_bwd_gpu import case, check_grads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_both(lib, q, k, v, dout, causal, scale):
    """The forward, then the atomic backward and the split backward on the
    same O and lse; returns ([dq, dk, dv] atomic, [dq, dk, dv] split) on the
    host as float32."""
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = lib.attention(qd, kd, vd, causal, scale)
    a = lib.attention_backward(qd, kd, vd, o, lse, dd, causal, scale, atomic=True)
    s = lib.attention_backward(qd, kd, vd, o, lse, dd, causal, scale)
    torch.cuda.synchronize()
    return ([x.float().cpu().numpy() for x in a], [x.float().cpu().numpy() for x in s])


def check_dkdv_match(label, a, s):
    """dK and dV come from the same products in the same order in both
    paths, so they agree bit for bit."""
    for name, x, y in zip(("dK", "dV"), a[1:], s[1:]):
        diff = float(np.abs(x.astype(np.float64) - y).max())
        assert np.array_equal(x, y), f"{label} {name}: atomic and split differ by {diff:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 77, 128, 129, 300, 1000])
def test_atomic_backward_ragged(gpu_lib, T, causal, dtype):
    """Two sequences, three heads, lengths around and between the 64-query
    tiles and 128-key blocks."""
    q, k, v, dout = case(2, 3, T, dtype, 4000 + T)
    flush_print(f"[gpu] atomic backward {dtype} T={T} causal={causal}")
    a, s = run_both(gpu_lib, q, k, v, dout, causal, 0.125)
    want = oracle.attention_backward(q, k, v, dout, causal, 0.125)
    check_grads(f"atomic {dtype} T={T} causal={causal}", a, want)
    check_dkdv_match(f"{dtype} T={T} causal={causal}", a, s)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_atomic_backward_scales(gpu_lib, scale):
    """Negative, zero and larger scales: the sign enters S, and scale
    multiplies dK in the main kernel and dQ in the last one."""
    q, k, v, dout = case(1, 2, 200, "bf16", 4100)
    flush_print(f"[gpu] atomic backward scale={scale}")
    a, s = run_both(gpu_lib, q, k, v, dout, True, scale)
    want = oracle.attention_backward(q, k, v, dout, True, scale)
    check_grads(f"atomic scale={scale}", a, want)
    check_dkdv_match(f"scale={scale}", a, s)


def test_atomic_backward_reuses_workspace(gpu_lib):
    """The call zeroes its own float32 dQ copy: two calls on one workspace
    give the same dQ up to the atomics' order (a missing clear would double
    it), and dK, dV bit for bit."""
    q, k, v, dout = (x.to(DEV) for x in case(2, 2, 333, "bf16", 4300))
    o, lse = gpu_lib.attention(q, k, v, True, 0.125)
    ws = torch.empty(gpu_lib.attn_bwd_atomic_workspace_bytes(2, 2, 333), dtype=torch.uint8,
                     device=DEV)
    outs = []
    for _ in range(2):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        gpu_lib.attn_bwd_atomic_stream(q, k, v, o, dout, lse, dq, dk, dv, ws, True, 0.125)
        torch.cuda.synchronize()
        outs.append([x.float().cpu().numpy() for x in (dq, dk, dv)])
    (dq1, dk1, dv1), (dq2, dk2, dv2) = outs
    scale = max(1.0, float(np.abs(dq1).max()))
    assert float(np.abs(dq1 - dq2).max()) <= 1e-2 * scale
    assert np.array_equal(dk1, dk2) and np.array_equal(dv1, dv2)


def test_atomic_backward_metric_workload_slices(gpu_lib):
    """The 4 x 12 x 8192 bf16 causal workload: the whole pass on the GPU, the
    oracle on two slices (the first and the last), every element of them."""
    q, k, v, dout = case(4, 12, 8192, "bf16", 2001)
    flush_print("[gpu] atomic backward 4x12x8192 bf16 causal")
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = gpu_lib.attention(qd, kd, vd, True, 0.125)
    got = gpu_lib.attention_backward(qd, kd, vd, o, lse, dd, True, 0.125, atomic=True)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in got]
    sl = np.array([0, 47])
    want = oracle.attention_backward(q, k, v, dout, True, 0.125, slices=sl)
    got_sl = [g.reshape(48, 8192, 64)[sl] for g in got]
    check_grads("atomic 4x12x8192 slices 0,47", got_sl, want)


def test_atomic_backward_invalid(gpu_lib):
    """Argument errors come back as status codes with nothing enqueued."""
    q, k, v, dout = (x.to(DEV) for x in case(1, 1, 64, "bf16", 4400))
    o, lse = gpu_lib.attention(q, k, v, True, 0.125)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = gpu_lib.attn_bwd_atomic_workspace_bytes(1, 1, 64)
    short = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.attn_bwd_atomic_stream(q, k, v, o, dout, lse, dq, dk, dv, short, True, 0.125)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.attn_bwd_atomic_stream(q, k, v, o, dout, lse, dq, dk, dv, ws, True,
                                       float("nan"))
