"""The no-allocation decode entry point (attn_decode_noalloc_stream) against
the workspace entry point (attn_decode_stream) and the oracle, through the C
ABI: two calls in a row on one GPU, the second with a smaller input, so the
shared scratch's counters and partials are reused after a call has left them
behind."""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = 2e-2


def flush_print(*a):
    print(*a, flush=True)


def run_both(lib, B, H, Tq, Tk, D, dtype, causal, seed):
    q, k, v = make_qkv(B, H, Tk, D, dtype, seed)
    q = q[:, :, Tk - Tq:].contiguous()
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o_ws, o_na = torch.empty_like(qd), torch.empty_like(qd)
    l_ws = torch.empty((B, H, Tq), dtype=torch.float32, device=DEV)
    l_na = torch.empty_like(l_ws)
    ws = torch.empty(lib.attn_decode_workspace_bytes(B, H, Tq, Tk, D), dtype=torch.uint8,
                     device=DEV)
    flush_print(f"[gpu] decode noalloc vs workspace B={B} H={H} Tq={Tq} Tk={Tk} D={D} "
                f"{dtype} causal={causal}")
    lib.attn_decode_stream(qd, kd, vd, o_ws, l_ws, ws, causal, D ** -0.5)
    lib.attn_decode_noalloc_stream(qd, kd, vd, o_na, l_na, causal, D ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_kv(q, k, v, causal, D ** -0.5)
    got_o, got_l = o_na.float().cpu().numpy(), l_na.cpu().numpy()
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    d_entry = float((o_na.float() - o_ws.float()).abs().max())
    d_lse = float((l_na - l_ws).abs().max())
    d_oracle = float(np.abs(got_o - ro).max())
    d_oracle_lse = float(np.abs(got_l - rl).max())
    flush_print(f"      vs attn_decode_stream max|dO| {d_entry:.2e} max|dlse| {d_lse:.2e}; "
                f"vs oracle {d_oracle:.2e} / {d_oracle_lse:.2e}")
    assert d_entry <= TOL and d_lse <= TOL
    assert d_oracle <= TOL and d_oracle_lse <= TOL


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (32, "f16")])
def test_noalloc_matches_workspace_entry_twice(gpu_lib, D, dtype):
    # a split plan with several key ranges per tile, then a smaller one
    run_both(gpu_lib, 4, 12, 1, 8192, D, dtype, True, 3101 + D)
    run_both(gpu_lib, 1, 3, 5, 700, D, dtype, True, 3201 + D)


def test_noalloc_single_split_and_full_mask(gpu_lib):
    # enough tiles that the plan keeps one key range per tile (the output is
    # written by the split itself), then a small non-causal call
    run_both(gpu_lib, 8, 40, 40, 256, 64, "bf16", True, 3301)
    run_both(gpu_lib, 2, 2, 3, 100, 64, "bf16", False, 3302)
