"""Seeded synthetic inputs for attention, shared by the tests, the benchmark
and the smoke check.

This module holds no attention arithmetic: it only draws numbers, casts them
to the storage dtype and picks row samples. Both the GPU path and the oracle
receive what it produces; neither is imported here.

Recipe (every config): ``torch.Generator('cpu').manual_seed(seed)``, then
``torch.randn`` in float32 for q, k and v in that order, shaped
[B, H, T, D], then a round-to-nearest-even cast to the storage dtype. The
pages test on seeded random tensors of this shape ("Flash attention in
PyTorch, then in Triton", section "Attention by hand"); the named workloads
below follow the shapes that page and the page "attention.cu" run.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention problem: layout [B, H, T, D], scale 1/sqrt(D)."""
    name: str
    B: int
    H: int
    T: int
    D: int
    causal: bool
    dtype: str  # "f32" | "bf16" | "f16"
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.T

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["scale"] = self.scale
        return d


def _wl(name, B, H, T, causal, dtype, seed, D=64):
    return Workload(name, B, H, T, D, causal, dtype, seed)


# The five workloads. Seeds are fixed per workload and length so every run
# (test, bench, smoke) sees the same numbers.
WORKLOADS = {
    # one head, non-causal, fp32, the first case of "attention.cu"
    "single_head_n256_f32": _wl("single_head_n256_f32", 1, 1, 256, False,
                                "f32", 1001),
    # one head, non-causal, fp32, the two larger cases of "attention.cu"
    "single_head_n1024_f32": _wl("single_head_n1024_f32", 1, 1, 1024, False,
                                 "f32", 1002),
    "single_head_n4096_f32": _wl("single_head_n4096_f32", 1, 1, 4096, False,
                                 "f32", 1003),
    # causal fp32, two sequences of three heads, the test lengths of
    # "Flash attention in PyTorch, then in Triton" (section "Attention by hand")
    **{f"causal_b2h3_t{T}_f32": _wl(f"causal_b2h3_t{T}_f32", 2, 3, T, True,
                                    "f32", 1100 + T)
       for T in (1, 100, 256, 1000)},
    # causal bf16, GPT-2-small-shaped: 4 sequences x 12 heads x 8192 tokens
    "gpt2s_b4h12_t8192_bf16": _wl("gpt2s_b4h12_t8192_bf16", 4, 12, 8192, True,
                                  "bf16", 2001),
    # causal long context, bf16, one sequence of 16 heads
    "long_b1h16_t32768_bf16": _wl("long_b1h16_t32768_bf16", 1, 16, 32768,
                                  True, "bf16", 3001),
    "long_b1h16_t131072_bf16": _wl("long_b1h16_t131072_bf16", 1, 16, 131072,
                                   True, "bf16", 3002),
}

# The metric's workload: causal, d = 64, bf16, T = 8192.
METRIC_WORKLOAD = "gpt2s_b4h12_t8192_bf16"


def make_qkv(B: int, H: int, T: int, D: int, dtype: str, seed: int):
    """Seeded q, k, v as CPU tensors of the storage dtype, shape [B,H,T,D]."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, H, T, D)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x.to(DTYPES[dtype]).contiguous())
    return tuple(out)


def make_gated(B: int, T: int, H: int, D: int, seed: int):
    """Seeded inputs of the gated linear recurrence as float32 CPU tensors
    [B, T, H, D]: q, k, v standard normal and the gate a logistic sigmoid of
    a standard normal draw, so every gate lies in (0, 1) (the input structure
    of the POPCORNBENCH transcript "Kimi-K2.6 l2 p24")."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, T, H, D)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    gate = torch.sigmoid(torch.randn(shape, generator=g, dtype=torch.float32))
    return q.contiguous(), k.contiguous(), v.contiguous(), gate.contiguous()


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.H, w.T, w.D, w.dtype, w.seed)


def late_spike_qkv(T: int, D: int = 64, dtype: str = "f32", spike: float = 3.0):
    """Deterministic one-head inputs [1, 1, T, D] with no tile-aligned
    pattern and one late key amplified, so a running maximum still grows on
    the final key tile.

    The idea (residues with periods that divide no tile size, plus one key
    near the end scaled up) is the stress input of the page "attention.cu";
    the residues, offsets and step sizes here are this module's own.
    """
    i = np.arange(T, dtype=np.int64)[:, None]
    e = np.arange(D, dtype=np.int64)[None, :]
    q = (((i * 29 + e * 5) % 101) - 50).astype(np.float32) * np.float32(0.0185)
    k = (((i * 19 + e * 13) % 89) - 44).astype(np.float32) * np.float32(0.0207)
    v = (((i * 11 + e * 7) % 79) - 39).astype(np.float32) * np.float32(0.0123)
    late = max(T - 3, 0)
    k[late] *= np.float32(spike)
    cast = DTYPES[dtype]
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).reshape(1, 1, T, D)
                 .to(cast).contiguous() for x in (q, k, v))


def sample_rows(B: int, H: int, T: int, n: int, seed: int,
                boundaries=(64, 128, 256)) -> np.ndarray:
    """Up to n distinct flat row ids (b * H + h) * T + t, drawn without
    replacement by a seeded generator, always including t = 0, t = T - 1 and
    the rows on both sides of each tile boundary in `boundaries` (for the
    first and last (b, h) slices). Sorted ascending."""
    total = B * H * T
    if n >= total:
        return np.arange(total, dtype=np.int64)
    forced = set()
    for slice_id in {0, B * H - 1}:
        base = slice_id * T
        for t in (0, T - 1):
            forced.add(base + t)
        for bnd in boundaries:
            for t in (bnd - 1, bnd):
                if 0 <= t < T:
                    forced.add(base + t)
    forced = sorted(forced)[:n]
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    need = n - len(forced)
    chosen = set(forced)
    while need > 0:
        cand = rng.integers(0, total, size=2 * need + 16, dtype=np.int64)
        for c in cand.tolist():
            if c not in chosen:
                chosen.add(c)
                need -= 1
                if need == 0:
                    break
    return np.array(sorted(chosen), dtype=np.int64)
