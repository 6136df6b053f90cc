"""flash_attention, the autograd function of "Flash attention in PyTorch,
then in Triton" (section "Backwards, and training with it"), on this
library's kernels: the output and the gradients torch.autograd computes
through it against the double oracle, bit for bit against the direct entry
points, under autocast from float32 leaves, with the atomic backward, and
the float32 backward refused."""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd import AttnError
from online_softmax_amd.inputs import make_qkv
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def close(name, got, want, bound):
    got = np.asarray(got, np.float64)
    err = float(np.abs(got - want).max())
    flush_print(f"    {name}: max|d| {err:.3e} (bound {bound:.2e})")
    assert np.all(np.isfinite(got)) and err <= bound, name


@pytest.mark.parametrize("atomic", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_autograd_matches_oracle_and_entry_points(gpu_lib, causal, atomic):
    B, H, T, D = 1, 2, 300, 64
    q, k, v = make_qkv(B, H, T, D, "bf16", 9100)
    (dout,) = make_qkv(B, H, T, D, "bf16", 9101)[:1]
    qd, kd, vd = (x.to(DEV).requires_grad_() for x in (q, k, v))
    dd = dout.to(DEV)
    flush_print(f"[gpu] flash_attention causal={causal} atomic={atomic}")
    o = gpu_lib.flash_attention(qd, kd, vd, causal=causal, atomic=atomic)
    grads = torch.autograd.grad(o, (qd, kd, vd), dd)
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, causal, D ** -0.5)
    close("O", o.detach().float().cpu().numpy(), ro, TOL)
    want = oracle.attention_backward(q, k, v, dout, causal, D ** -0.5)
    for name, g, w in zip(("dQ", "dK", "dV"), grads, want):
        w = np.asarray(w, np.float64)
        close(name, g.float().cpu().numpy().reshape(w.shape), w, TOL * max(1.0, np.abs(w).max()))
    # the same kernels through the direct entry points
    o2, lse2 = gpu_lib.attention(qd.detach(), kd.detach(), vd.detach(), causal, D ** -0.5)
    direct = gpu_lib.attention_backward(qd.detach(), kd.detach(), vd.detach(), o2, lse2, dd,
                                        causal, D ** -0.5, atomic=atomic)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for name, g, h in zip(("dQ", "dK", "dV"), grads, direct):
        if atomic and name == "dQ":  # float32 atomic adds land in any order
            assert (g.float() - h.float()).abs().max().item() <= 1e-2
        else:
            assert torch.equal(g, h), name


def test_autocast_from_float32_leaves(gpu_lib):
    """Under autocast the function casts q, k, v to autocast's dtype (bf16
    here), as the page's function does; the gradients come back to the
    float32 leaves through the casts."""
    B, H, T, D = 1, 2, 200, 64
    q, k, v = make_qkv(B, H, T, D, "f32", 9200)
    (dout,) = make_qkv(B, H, T, D, "bf16", 9201)[:1]
    qd, kd, vd = (x.to(DEV).requires_grad_() for x in (q, k, v))
    flush_print("[gpu] flash_attention under autocast (bf16) from float32 leaves")
    with torch.autocast("cuda", dtype=torch.bfloat16):
        o = gpu_lib.flash_attention(qd, kd, vd)
    assert o.dtype == torch.bfloat16
    grads = torch.autograd.grad(o, (qd, kd, vd), dout.to(DEV))
    torch.cuda.synchronize()
    assert all(g.dtype == torch.float32 for g in grads)
    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    ro, _ = oracle.attention(qb, kb, vb, True, D ** -0.5)
    close("O", o.detach().float().cpu().numpy(), ro, TOL)
    want = oracle.attention_backward(qb, kb, vb, dout, True, D ** -0.5)
    for name, g, w in zip(("dQ", "dK", "dV"), grads, want):
        w = np.asarray(w, np.float64)
        close(name, g.cpu().numpy().reshape(w.shape), w, TOL * max(1.0, np.abs(w).max()))


def test_float32_forward_and_refused_backward(gpu_lib):
    B, H, T, D = 1, 2, 100, 64
    q, k, v = make_qkv(B, H, T, D, "f32", 9300)
    qd, kd, vd = (x.to(DEV).requires_grad_() for x in (q, k, v))
    o = gpu_lib.flash_attention(qd, kd, vd)
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, True, D ** -0.5)
    close("O f32", o.detach().cpu().numpy(), ro, 1e-5)
    with pytest.raises(AttnError, match="bf16 or f16"):
        torch.autograd.grad(o, (qd, kd, vd), torch.ones_like(o))
