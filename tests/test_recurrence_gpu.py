"""GPU parity of the gated linear recurrence (attn_gated_recurrence_stream,
float32) against the double oracle on the same seeded inputs.

Tolerance, per element y[b, t, h, j]: |delta| <= 2 (D + t + 2) 2^-24 A[b, t,
h, j] + 1e-30, where A is the recurrence run by the oracle on |q|, |k|, |v|
and the same (positive) gates: the sum of the magnitudes of every term that
makes y. Float32 forms each state element by t + 1 multiply-adds (each
rounding the running sum once, the product k v once more; older errors are
scaled down by the gates) and the readout by D products summed, so the
first-order forward error bound is (D + t + 2) u A with u = 2^-24; the
factor 2 covers second-order terms. Any non-finite output fails.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_gated
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def run(lib, q, k, v, g):
    y = lib.gated_recurrence(*(x.to(DEV) for x in (q, k, v, g)))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(label, got, q, k, v, g):
    want = oracle.gated_recurrence(q, k, v, g)
    mag = oracle.gated_recurrence(q.abs(), k.abs(), v.abs(), g)
    T, D = q.shape[1], q.shape[3]
    t = np.arange(T, dtype=np.float64).reshape(1, T, 1, 1)
    bound = 2.0 * (D + t + 2) * U * mag + 1e-30
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - want)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    flush_print(f"    {label}: max|d| = {err.max():.3e}, max |d| / bound = "
                f"{ratio.max():.3f}")
    assert ratio.max() <= 1.0, (f"{label}: at {np.unravel_index(worst, err.shape)} got "
                                f"{got.flat[worst]!r} want {want.flat[worst]!r} bound "
                                f"{bound.flat[worst]:.3e}")


def test_page_size(gpu_lib):
    """Two sequences, four heads, 128 steps, head dimension 24: the size the
    page's workload uses; three seeds."""
    for seed in (1, 2, 3):
        q, k, v, g = make_gated(2, 128, 4, 24, seed=7000 + seed)
        flush_print(f"[gpu] recurrence 2x128x4x24 seed {seed}")
        check(f"page size seed {seed}", run(gpu_lib, q, k, v, g), q, k, v, g)


@pytest.mark.parametrize("D", [1, 7, 8, 9, 16, 24, 33, 40, 57, 64])
@pytest.mark.parametrize("T", [1, 5, 17, 300])
def test_dims_and_lengths(gpu_lib, D, T):
    """Few slices (the per-wave kernel): every register-block size
    (ceil(D / 8) rows per lane, 1..8), head dims that leave lanes idle, and
    lengths that end mid-block."""
    q, k, v, g = make_gated(2, T, 3, D, seed=7100 + 100 * D + T)
    flush_print(f"[gpu] recurrence D={D} T={T}")
    check(f"D={D} T={T}", run(gpu_lib, q, k, v, g), q, k, v, g)


@pytest.mark.parametrize("D", [1, 7, 9, 24, 33, 57, 64])
@pytest.mark.parametrize("T", [1, 17, 300])
def test_many_slices(gpu_lib, D, T):
    """128 (batch, head) slices: the workgroup kernel (inputs staged through
    LDS in blocks of steps), every register-row count, lengths that end
    mid-block; every element checked."""
    q, k, v, g = make_gated(2, T, 64, D, seed=7400 + 100 * D + T)
    flush_print(f"[gpu] recurrence 2x{T}x64x{D}")
    check(f"2x{T}x64x{D}", run(gpu_lib, q, k, v, g), q, k, v, g)


def test_unit_and_zero_gates(gpu_lib):
    """gate = 1 over 2048 steps (the state is a running sum and grows), and
    gate = 0 (only the current step counts)."""
    q, k, v, _ = make_gated(1, 2048, 2, 32, seed=7200)
    flush_print("[gpu] recurrence gate = 1, T = 2048")
    g = torch.ones_like(q)
    check("gate 1", run(gpu_lib, q, k, v, g), q, k, v, g)
    g = torch.zeros_like(q)
    flush_print("[gpu] recurrence gate = 0")
    check("gate 0", run(gpu_lib, q, k, v, g), q, k, v, g)


def test_throughput_shape_sampled(gpu_lib):
    """8 x 4096 x 32 x 64 (the throughput workload the benchmark times): the
    whole call on the GPU, the oracle on four (batch, head) slices."""
    B, T, H, D = 8, 4096, 32, 64
    q, k, v, g = make_gated(B, T, H, D, seed=7300)
    flush_print(f"[gpu] recurrence {B}x{T}x{H}x{D}")
    y = run(gpu_lib, q, k, v, g)
    assert np.all(np.isfinite(y))
    for b, h in ((0, 0), (3, 17), (7, 31), (5, 2)):
        sl = [x[b:b + 1, :, h:h + 1].contiguous() for x in (q, k, v, g)]
        check(f"slice b={b} h={h}", y[b:b + 1, :, h:h + 1], *sl)


def test_invalid_calls_raise(gpu_lib):
    q = torch.zeros(1, 4, 1, 65, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.gated_recurrence(q, q, q, q)
    q = torch.zeros(1, 4, 1, 8, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gpu_lib.gated_recurrence(q, q, q, q)
