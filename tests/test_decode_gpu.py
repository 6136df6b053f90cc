"""GPU parity of the decode path (attn_decode_stream: Tq new queries against
a Tk-token key/value cache, causal mask aligned to the bottom-right) against
the double oracle (oracle.attention_kv) on the same seeded 16-bit inputs.
Tolerance: the forward's, 2e-2 on O and lse (the kernel's arithmetic per key
tile is the forward's; the merge of the splits is exact up to float32
rounding). Any non-finite output fails."""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_qkv
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(lib, q, k, v, causal, scale):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = lib.attention_decode(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(label, got, want, bound=2e-2):
    for name, g, w in zip(("O", "lse"), got, want):
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        err = float(np.abs(g.astype(np.float64) - w).max())
        flush_print(f"    {label} {name}: max|d| = {err:.3e} (bound {bound})")
        assert err <= bound, f"{label} {name}: {err:.3e} > {bound}"


def inputs(B, H, Tq, Tk, dtype, seed, D=64):
    (q,) = make_qkv(B, H, Tq, D, dtype, seed)[:1]
    _, k, v = make_qkv(B, H, Tk, D, dtype, seed + 1)
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 77), (1, 1000), (7, 300), (32, 1024),
                                   (33, 100), (64, 64), (100, 4096)])
def test_decode_parity(gpu_lib, Tq, Tk, causal, dtype):
    q, k, v = inputs(2, 3, Tq, Tk, dtype, 5000 + Tq * 7 + Tk)
    flush_print(f"[gpu] decode {dtype} Tq={Tq} Tk={Tk} causal={causal}")
    got = run(gpu_lib, q, k, v, causal, 0.125)
    want = oracle.attention_kv(q, k, v, causal, 0.125)
    check(f"{dtype} Tq={Tq} Tk={Tk} causal={causal}", got, want)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_decode_scales(gpu_lib, scale):
    q, k, v = inputs(1, 4, 5, 777, "bf16", 5100)
    flush_print(f"[gpu] decode scale={scale}")
    check(f"scale={scale}", run(gpu_lib, q, k, v, True, scale),
          oracle.attention_kv(q, k, v, True, scale))


def test_decode_bench_workload(gpu_lib):
    """The decode workload of the bench: one new token per sequence against
    an 8192-token cache, 4 sequences x 12 heads, bf16; every row checked."""
    q, k, v = inputs(4, 12, 1, 8192, "bf16", 2101)
    flush_print("[gpu] decode 4x12 Tq=1 Tk=8192")
    check("4x12 Tq=1 Tk=8192", run(gpu_lib, q, k, v, True, 0.125),
          oracle.attention_kv(q, k, v, True, 0.125))


def test_decode_last_rows_match_the_forward(gpu_lib):
    """Decoding the last Tq tokens of a sequence equals those rows of the
    library's own causal forward over the whole sequence, to rounding."""
    q, k, v = make_qkv(1, 2, 300, 64, "bf16", 5200)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o_full, l_full = gpu_lib.attention(qd, kd, vd, True, 0.125)
    o_dec, l_dec = gpu_lib.attention_decode(qd[:, :, 260:].contiguous(), kd, vd, True, 0.125)
    torch.cuda.synchronize()
    d = (o_full[:, :, 260:].float() - o_dec.float()).abs().max().item()
    dl = (l_full[:, :, 260:] - l_dec).abs().max().item()
    flush_print(f"    decode vs forward: max|dO| {d:.3e} max|dlse| {dl:.3e}")
    assert d <= 2e-2 and dl <= 2e-2


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 1000), (7, 300), (33, 100), (100, 2049)])
def test_decode_head_dims(gpu_lib, Tq, Tk, causal, dtype, D):
    """Head dimensions 32 and 128: the same split and merge over tiles of D
    columns (D / 16 steps of S, D / 32 output tiles)."""
    q, k, v = inputs(2, 3, Tq, Tk, dtype, 5300 + Tq * 7 + Tk + D, D)
    flush_print(f"[gpu] decode D={D} {dtype} Tq={Tq} Tk={Tk} causal={causal}")
    got = run(gpu_lib, q, k, v, causal, 0.125)
    want = oracle.attention_kv(q, k, v, causal, 0.125)
    check(f"D={D} {dtype} Tq={Tq} Tk={Tk} causal={causal}", got, want)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_many_splits(gpu_lib, D):
    """One slice, one token, a 32768-token cache: 256 key ranges, so the
    merge runs its loop over the splits four times."""
    q, k, v = inputs(1, 1, 1, 32768, "bf16", 5400 + D, D)
    flush_print(f"[gpu] decode D={D} 1x1 Tq=1 Tk=32768")
    check(f"D={D} Tk=32768", run(gpu_lib, q, k, v, True, 1.0 / np.sqrt(D)),
          oracle.attention_kv(q, k, v, True, 1.0 / np.sqrt(D)))


def test_decode_d128_workload(gpu_lib):
    """One new token per sequence against an 8192-token cache, 4 sequences x
    12 heads at head dimension 128, bf16; every row checked."""
    q, k, v = inputs(4, 12, 1, 8192, "bf16", 2111, 128)
    flush_print("[gpu] decode D=128 4x12 Tq=1 Tk=8192")
    check("D=128 4x12 Tq=1 Tk=8192", run(gpu_lib, q, k, v, True, 0.125),
          oracle.attention_kv(q, k, v, True, 0.125))


@pytest.mark.parametrize("D", [32, 128])
def test_decode_last_rows_match_the_forward_head_dims(gpu_lib, D):
    """As above, against the forward of the same head dimension."""
    q, k, v = make_qkv(1, 2, 300, D, "f16", 5500 + D)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o_full, l_full = gpu_lib.attention(qd, kd, vd, True, 0.125)
    o_dec, l_dec = gpu_lib.attention_decode(qd[:, :, 250:].contiguous(), kd, vd, True, 0.125)
    torch.cuda.synchronize()
    d = (o_full[:, :, 250:].float() - o_dec.float()).abs().max().item()
    dl = (l_full[:, :, 250:] - l_dec).abs().max().item()
    flush_print(f"    D={D} decode vs forward: max|dO| {d:.3e} max|dlse| {dl:.3e}")
    assert d <= 2e-2 and dl <= 2e-2
