"""GPU parity of the backward pass: dQ, dK, dV from the HIP kernels (called
through the C ABI, after the library's own forward produced O and lse)
against the double oracle's gradients of the same seeded 16-bit inputs.

Tolerance, per gradient tensor of a case: max |delta| <= 2e-2 * max(1, max
|g|), g the oracle's gradient. The kernels round P and dS to the input's
16-bit type for the products (relative error up to 2^-9 each, bf16) and the
result once more, and they start from the forward's O rounded to that type
(delta) and its float32 lse; those errors are a few times 2^-9 of the
gradient's own scale, the same order as the forward's 2e-2 bound on an
output of magnitude about 1, so the bound is that figure relative to the
gradient's largest entry. Any non-finite output fails.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_qkv
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_backward(lib, q, k, v, dout, causal, scale):
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = lib.attention(qd, kd, vd, causal, scale)
    dq, dk, dv = lib.attention_backward(qd, kd, vd, o, lse, dd, causal, scale)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def check_grads(label, got, want):
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        g = np.asarray(g, np.float64).reshape(w.shape)
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite output"
        err = np.abs(g - w)
        scale = max(1.0, float(np.abs(w).max()))
        bound = 2e-2 * scale
        mx = float(err.max())
        rms = float(np.sqrt(np.mean(err ** 2)))
        flush_print(f"    {label} {name}: max|d| = {mx:.3e} rms {rms:.2e} "
                    f"(max|g| {np.abs(w).max():.3e}, bound {bound:.1e})")
        worst = int(np.argmax(err))
        assert mx <= bound, (f"{label} {name}: max|d| {mx:.3e} > {bound:.1e} at "
                             f"{np.unravel_index(worst, err.shape)}: got "
                             f"{g.flat[worst]!r} want {w.flat[worst]!r}")


def case(B, H, T, dtype, seed):
    q, k, v = make_qkv(B, H, T, 64, dtype, seed)
    (dout,) = make_qkv(B, H, T, 64, dtype, seed + 7)[:1]
    return q, k, v, dout


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 77, 128, 300, 1000])
def test_backward_ragged(gpu_lib, T, causal, dtype):
    """The page's test shapes (two sequences, three heads) at ragged lengths."""
    q, k, v, dout = case(2, 3, T, dtype, 4000 + T)
    flush_print(f"[gpu] backward {dtype} T={T} causal={causal}")
    got = gpu_backward(gpu_lib, q, k, v, dout, causal, 0.125)
    want = oracle.attention_backward(q, k, v, dout, causal, 0.125)
    check_grads(f"{dtype} T={T} causal={causal}", got, want)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_backward_scales(gpu_lib, scale):
    """Negative, zero and larger scales (the sign enters S and the final
    multiplication of dQ and dK)."""
    q, k, v, dout = case(1, 2, 200, "bf16", 4100)
    flush_print(f"[gpu] backward scale={scale}")
    got = gpu_backward(gpu_lib, q, k, v, dout, True, scale)
    want = oracle.attention_backward(q, k, v, dout, True, scale)
    check_grads(f"scale={scale}", got, want)


def test_backward_metric_workload_slices(gpu_lib):
    """The 4 x 12 x 8192 bf16 causal workload: the whole pass on the GPU, the
    oracle on two slices (the first and the last), every element of them."""
    q, k, v, dout = case(4, 12, 8192, "bf16", 2001)
    flush_print("[gpu] backward 4x12x8192 bf16 causal")
    got = gpu_backward(gpu_lib, q, k, v, dout, True, 0.125)
    sl = np.array([0, 47])
    want = oracle.attention_backward(q, k, v, dout, True, 0.125, slices=sl)
    got_sl = [g.reshape(48, 8192, 64)[sl] for g in got]
    check_grads("4x12x8192 slices 0,47", got_sl, want)


@pytest.mark.parametrize("T", [77, 300])
def test_bf16_gradients_within_twice_torch_cpu_error(gpu_lib, T):
    """The backward's own rule on its page ("Flash attention in PyTorch, then
    in Triton", section "Backwards, and training with it"): for each of dQ,
    dK and dV, our bf16 error against float64 is at most twice that of
    torch's own attention in bf16 (here torch's CPU kernel and its autograd),
    plus a tiny margin."""
    q, k, v, dout = case(2, 3, T, "bf16", 4200 + T)
    got = gpu_backward(gpu_lib, q, k, v, dout, True, 0.125)
    want = oracle.attention_backward(q, k, v, dout, True, 0.125)
    tq, tk, tv = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=0.125)
    theirs = [g.float().numpy() for g in torch.autograd.grad(out, (tq, tk, tv), dout)]
    for name, g, t, w in zip(("dQ", "dK", "dV"), got, theirs, want):
        ours_err = float(np.abs(np.asarray(g, np.float64).reshape(w.shape) - w).max())
        their_err = float(np.abs(t.astype(np.float64) - w).max())
        flush_print(f"    bf16 T={T} {name}: ours {ours_err:.3e} torch-cpu {their_err:.3e}")
        assert ours_err <= 2 * their_err + 1e-5, name
