"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed. The library allocates nothing and issues no memset or
synchronisation inside a call, so a call on the capturing stream records
its kernel launches and nothing else. Each graph is replayed several times
with the outputs poisoned and unrelated eager work between the replays, and
every replay must reproduce the eager call: bit for bit where the kernels
are deterministic (forward, decode, the two-kernel backward), and within
float32 rounding for dQ of the atomic backward, whose adds land in any
order.
"""
import pytest
import torch

from online_softmax_amd.inputs import make_qkv
from conftest import flush_print

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def replay_check(name, run, outs, exact=None):
    """run() enqueues one call on the current stream writing `outs`; exact[i]
    False allows float32 rounding differences for outs[i]."""
    exact = exact or [True] * len(outs)
    run()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    # warm up on a side stream (default priority), as capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for x in outs:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (x, r, ex) in enumerate(zip(outs, ref, exact)):
            if ex:
                assert torch.equal(x, r), f"{name}: replay {i}, output {j} differs"
            else:
                d = (x.float() - r.float()).abs().max().item()
                scale = max(1.0, r.float().abs().max().item())
                assert d <= 1e-2 * scale, f"{name}: replay {i}, output {j}: {d}"
        # unrelated eager work between replays
        junk = torch.randn(1 << 16, device=DEV).sum().item()
        assert junk == junk
    flush_print(f"    {name}: {REPLAYS} replays match the eager call")


@pytest.mark.parametrize("shape", [(4, 64, 300, True), (2, 3, 1000, True), (4, 12, 1024, False)],
                         ids=["w8", "w8s", "r128"])
def test_forward_graph_replay(gpu_lib, shape):
    B, H, T, causal = shape
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, T, 64, "bf16", 8100 + T))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    kernel = gpu_lib.attn_kernel_name(gpu_lib.attn_fused_kernel(B, H, T, 64, causal,
                                                                gpu_lib.ATTN_BF16))
    flush_print(f"[gpu] graph: forward {B}x{H}x{T} causal={causal} ({kernel})")
    replay_check("forward", lambda: gpu_lib.attn_fwd_stream(q, k, v, o, lse, causal, 0.125),
                 [o, lse])


@pytest.mark.parametrize("D", [64, 128])
def test_decode_graph_replay(gpu_lib, D):
    B, H, Tq, Tk = 2, 3, 1, 1000
    q = make_qkv(B, H, Tq, D, "bf16", 8200)[0].to(DEV)
    _, k, v = (x.to(DEV) for x in make_qkv(B, H, Tk, D, "bf16", 8201))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=DEV)
    ws = torch.empty(gpu_lib.attn_decode_workspace_bytes(B, H, Tq, Tk, D), dtype=torch.uint8,
                     device=DEV)
    flush_print(f"[gpu] graph: decode D={D} (workspace, then no allocation)")
    replay_check("decode", lambda: gpu_lib.attn_decode_stream(q, k, v, o, lse, ws, True, 0.125),
                 [o, lse])
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    replay_check("decode without allocation",
                 lambda: gpu_lib.attn_decode_noalloc_stream(q, k, v, o2, lse2, True, 0.125),
                 [o2, lse2])
    assert torch.equal(o2, o)


@pytest.mark.parametrize("atomic", [False, True])
def test_backward_graph_replay(gpu_lib, atomic):
    B, H, T = 1, 2, 300
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, T, 64, "bf16", 8300))
    dout = make_qkv(B, H, T, 64, "bf16", 8301)[0].to(DEV)
    o, lse = gpu_lib.attention(q, k, v, True, 0.125)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    need = (gpu_lib.attn_bwd_atomic_workspace_bytes if atomic
            else gpu_lib.attn_bwd_workspace_bytes)(B, H, T)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    entry = gpu_lib.attn_bwd_atomic_stream if atomic else gpu_lib.attn_bwd_stream
    flush_print(f"[gpu] graph: backward atomic={atomic}")
    replay_check("backward", lambda: entry(q, k, v, o, dout, lse, dq, dk, dv, ws, True, 0.125),
                 [dq, dk, dv], exact=[not atomic, True, True])
