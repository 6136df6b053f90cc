"""GPU parity of the forward pass at head dimensions 32 and 128 (the 16-bit
fused kernels built per head dimension) against the double oracle, which
takes any D, on the same seeded rounded inputs.

Tolerance as for D = 64 in 16 bits: max |delta| <= 2e-2 on every checked
element of O and of lse. The kernels round the weights p to the input's
type for the P V product and the output once more; neither error depends on
D, while each score's float32 accumulation error grows only with sqrt(D)
times 2^-24 of the score's magnitude, far below the bound. Any non-finite
output fails.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import late_spike_qkv, make_qkv, sample_rows
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def fused(lib, q, k, v, causal, scale):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = lib.attention(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def assert_close(name, got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    worst = int(np.argmax(err)) if err.size else 0
    flush_print(f"    {name}: max|d| = {mx:.3e} (bound {TOL:.0e})")
    assert mx <= TOL, (f"{name}: max|d| {mx:.3e} at flat index {worst}: got "
                       f"{got.flat[worst]!r} want {want.flat[worst]!r}")


def check(lib, q, k, v, causal, scale, label):
    flush_print(f"[gpu] {label}: shape {tuple(q.shape)} {q.dtype} causal={causal}")
    o, lse = fused(lib, q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal, scale)
    assert_close(label + " O", o, ro)
    assert_close(label + " lse", lse, rl)


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 77, 128, 300, 1000])
def test_ragged(gpu_lib, D, dtype, causal, T):
    """Two sequences of three heads at ragged lengths: one partial tile, one
    exact query tile, several tiles with a ragged tail."""
    q, k, v = make_qkv(2, 3, T, D, dtype, 6000 + T + D)
    check(gpu_lib, q, k, v, causal, 1.0 / np.sqrt(D), f"D{D} {dtype} T={T}")


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_scales(gpu_lib, D, scale):
    """A negative scale (Q negated inside), zero (uniform weights) and a
    larger one."""
    q, k, v = make_qkv(1, 2, 200, D, "bf16", 6100 + D)
    check(gpu_lib, q, k, v, True, scale, f"D{D} scale={scale}")


@pytest.mark.parametrize("D", [32, 128])
def test_late_spike_and_rising_scores(gpu_lib, D):
    """A key amplified near the end, and keys scaled up steadily along the
    sequence: the running maximum still moves on late tiles."""
    q, k, v = late_spike_qkv(1000, D, "bf16")
    check(gpu_lib, q, k, v, True, 0.125, f"D{D} late spike")
    T = 2048
    q, k, v = make_qkv(1, 2, T, D, "f32", 6200 + D)
    k = (k * torch.linspace(1.0, 6.0, T).reshape(1, 1, T, 1)).to(torch.bfloat16)
    q, v = q.to(torch.bfloat16), v.to(torch.bfloat16)
    check(gpu_lib, q, k, v, False, 0.125, f"D{D} rising")


@pytest.mark.parametrize("D", [32, 128])
def test_single_token_returns_v(gpu_lib, D):
    """T = 1: the one weight is 1, so O = V exactly (one rounding of V, which
    is already 16-bit) and lse is the score."""
    q, k, v = make_qkv(3, 2, 1, D, "bf16", 6300 + D)
    o, lse = fused(gpu_lib, q, k, v, True, 0.2)
    assert np.array_equal(o, v.float().numpy())
    ro, rl = oracle.attention(q, k, v, True, 0.2)
    assert_close(f"D{D} T=1 lse", lse, rl)


@pytest.mark.parametrize("D", [32, 128])
def test_metric_shape_sampled(gpu_lib, D):
    """4 x 12 x 8192 bf16 causal at this head dimension, in the launch the
    benchmark times: the whole pass on the GPU, the oracle on 2048 sampled
    rows (tile boundaries and both ends of the first and last slices
    included)."""
    B, H, T = 4, 12, 8192
    q, k, v = make_qkv(B, H, T, D, "bf16", 6400 + D)
    flush_print(f"[gpu] D{D} {B}x{H}x{T} bf16 causal")
    o, lse = fused(gpu_lib, q, k, v, True, 1.0 / np.sqrt(D))
    rows = sample_rows(B, H, T, 2048, 6500 + D, boundaries=(64, 128, 256, T // 2))
    ro, rl = oracle.attention(q, k, v, True, 1.0 / np.sqrt(D), rows=rows)
    assert_close(f"D{D} sampled O", o.reshape(-1, D)[rows], ro)
    assert_close(f"D{D} sampled lse", lse.reshape(-1)[rows], rl)
    assert np.all(np.isfinite(o)), "non-finite output somewhere"
