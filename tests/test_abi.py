"""CPU tests of the C ABI (no GPU): the library loads and exports every
symbol include/attn.h declares; invalid arguments return the documented
status before any HIP call; the traffic and FLOP arithmetic matches closed
forms and the figures the pages state.

Every compute call made here is INVALID by construction (each carries at
least one bad argument), so it is rejected before a launch; none of these
tests can start a kernel, on any machine."""
import json
import math
import os
import re

import pytest

import online_softmax_amd as osa
from online_softmax_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden",
                                     "page_figures.json")))
FAKE = 0x10000  # 16-byte aligned, never dereferenced (every call is invalid)


@pytest.fixture(scope="module")
def lib():
    return osa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"
    assert sorted(binding.EXPORTS) == names


def test_status_strings(lib):
    for st in (0, -1, -2, -3, 42):
        assert isinstance(osa.attn_status_string(st), str)
    assert osa.attn_status_string(-1) == "invalid argument"
    assert osa.attn_last_hip_error() == 0


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, T=8, D=64,
        causal=1, scale=0.125, dtype=1, stream=None):
    return lib.attn_fwd_stream(q, k, v, o, lse, B, H, T, D, causal,
                               scale, dtype, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1),
    (dict(o=None), -1),
    (dict(B=0), -1), (dict(H=0), -1), (dict(T=0), -1), (dict(T=-5), -1),
    (dict(D=0), -1), (dict(D=96), -2), (dict(D=16), -2), (dict(D=256), -2),
    (dict(D=32, dtype=0), -2), (dict(D=128, dtype=0), -2),  # float32: D = 64 only
    (dict(dtype=3), -1), (dict(dtype=-1), -1),
    (dict(scale=math.inf), -1), (dict(scale=math.nan), -1),
    (dict(scale=3e38), -1),  # |scale| * log2(e) overflows float
    (dict(q=FAKE + 8), -1), (dict(o=FAKE + 4), -1), (dict(lse=FAKE + 2), -1),
    (dict(B=65536, H=65536), -2),   # B*H beyond int32
    (dict(B=4096, H=2048, T=256), -2),  # grid beyond one launch
])
def test_fused_rejects_invalid(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.attn_fwd(*[kw.get(n, d) for n, d in
                          (("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE),
                           ("lse", FAKE), ("B", 1), ("H", 1), ("T", 8),
                           ("D", 64), ("causal", 1), ("scale", 0.125),
                           ("dtype", 1))]) == status


def naive(lib, q=FAKE, ws=FAKE, ws_bytes=1 << 40, B=1, H=1, T=8, D=64,
          dtype=0, scale=0.125, lse=FAKE):
    return lib.attn_naive_fwd(q, FAKE, FAKE, FAKE, lse, ws, ws_bytes, B, H, T,
                              D, 1, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(ws=None), -1), (dict(T=0), -1),
    (dict(D=80), -2), (dict(D=32), -2), (dict(D=128), -2), (dict(dtype=1), -2), (dict(dtype=2), -2),
    (dict(dtype=7), -1), (dict(scale=math.nan), -1), (dict(ws=FAKE + 4), -1),
    (dict(ws_bytes=100), -1), (dict(lse=FAKE + 1), -1),
    (dict(B=70000, T=8), -2),  # grid y/z beyond 65535
])
def test_naive_rejects_invalid(lib, kw, status):
    assert naive(lib, **kw) == status


def bwd(lib, entry, q=FAKE, o=FAKE, lse=FAKE, dq=FAKE, ws=FAKE, ws_bytes=1 << 40, B=1,
        H=1, T=8, D=64, dtype=1, scale=0.125):
    return getattr(lib, entry)(q, FAKE, FAKE, o, FAKE, lse, dq, FAKE, FAKE, ws,
                               ws_bytes, B, H, T, D, 1, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(dq=None), -1), (dict(ws=None), -1), (dict(T=0), -1), (dict(B=0), -1),
    (dict(D=128), -2), (dict(D=32), -2), (dict(dtype=0), -2), (dict(dtype=5), -1),
    (dict(scale=math.nan), -1), (dict(scale=3e38), -1),
    (dict(q=FAKE + 8), -1), (dict(dq=FAKE + 2), -1), (dict(ws=FAKE + 4), -1),
    (dict(lse=FAKE + 2), -1), (dict(ws_bytes=16), -1),
    (dict(B=4096, H=2048, T=256), -2),  # grid beyond one launch
    (dict(T=1 << 25), -2),  # one slice over 4 GiB
])
@pytest.mark.parametrize("entry", ["attn_bwd_stream", "attn_bwd_atomic_stream"])
def test_bwd_rejects_invalid(lib, entry, kw, status):
    assert bwd(lib, entry, **kw) == status


def test_bwd_atomic_workspace_bytes(lib):
    """The split backward's row workspace (attn_bwd_workspace_bytes)
    followed by the float32 copy of dQ; a workspace one byte short is
    refused."""
    for B, H, T in [(1, 1, 1), (2, 3, 1000), (4, 12, 8192)]:
        rows = osa.attn_bwd_workspace_bytes(B, H, T)
        assert rows == 2 * -(-B * H * T * 4 // 256) * 256
        need = osa.attn_bwd_atomic_workspace_bytes(B, H, T)
        assert need == rows + B * H * T * 64 * 4
        assert bwd(lib, "attn_bwd_atomic_stream", B=B, H=H, T=T, ws_bytes=need - 1) == -1
    assert osa.attn_bwd_atomic_workspace_bytes(0, 1, 1) == 0
    assert osa.attn_bwd_atomic_workspace_bytes(1 << 30, 1 << 30, 1 << 30) == 0


def test_bwd_workspace_and_flops():
    for B, H, T in [(1, 1, 1), (2, 3, 1000), (4, 12, 8192)]:
        assert osa.attn_bwd_workspace_bytes(B, H, T) == 2 * -(-B * H * T * 4 // 256) * 256
    assert osa.attn_bwd_workspace_bytes(0, 1, 1) == 0
    assert osa.attn_bwd_workspace_bytes(1 << 30, 1 << 30, 1 << 30) == 0
    # five products to the forward's two
    assert osa.attn_bwd_flops(4, 12, 8192, 64, True) == 5.0 * 4 * 12 * 8192 ** 2 * 64
    assert osa.attn_bwd_flops(1, 1, 10, 64, False) == 2.5 * 4 * 100 * 64


def dec(lib, q=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40, B=1, H=1, Tq=1, Tk=8,
        D=64, dtype=1, scale=0.125):
    return lib.attn_decode_stream(q, FAKE, FAKE, FAKE, lse, ws, ws_bytes, B, H, Tq, Tk,
                                  D, 1, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(ws=None), -1), (dict(Tq=0), -1), (dict(Tk=0), -1),
    (dict(Tq=9, Tk=8), -1), (dict(B=0), -1), (dict(D=96), -2), (dict(D=16), -2),
    (dict(D=256), -2), (dict(dtype=0), -2),
    (dict(dtype=9), -1), (dict(scale=math.inf), -1), (dict(q=FAKE + 8), -1),
    (dict(ws=FAKE + 4), -1), (dict(lse=FAKE + 2), -1), (dict(ws_bytes=16), -1),
    (dict(Tk=1 << 25), -2),  # one cache slice over 4 GiB
])
def test_decode_rejects_invalid(lib, kw, status):
    assert dec(lib, **kw) == status


def dec_noalloc(lib, q=FAKE, lse=FAKE, B=1, H=1, Tq=1, Tk=8, D=64, dtype=1, scale=0.125):
    return lib.attn_decode_noalloc_stream(q, FAKE, FAKE, FAKE, lse, B, H, Tq, Tk, D, 1,
                                          scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(Tq=0), -1), (dict(Tk=0), -1),
    (dict(Tq=9, Tk=8), -1), (dict(B=0), -1), (dict(D=96), -2), (dict(D=16), -2),
    (dict(dtype=0), -2), (dict(dtype=9), -1), (dict(scale=math.inf), -1),
    (dict(q=FAKE + 8), -1), (dict(lse=FAKE + 2), -1),
    (dict(Tk=1 << 25), -2),  # one cache slice over 4 GiB
])
def test_decode_noalloc_rejects_invalid(lib, kw, status):
    """Every check runs before the first HIP call (none reaches the device)."""
    assert dec_noalloc(lib, **kw) == status


def rec(lib, q=FAKE, y=FAKE, B=1, T=8, H=1, D=24):
    return lib.attn_gated_recurrence_stream(q, FAKE, FAKE, FAKE, y, B, T, H, D, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(y=None), -1), (dict(B=0), -1), (dict(T=0), -1),
    (dict(H=-1), -1), (dict(D=0), -1), (dict(D=65), -2), (dict(D=128), -2),
    (dict(q=FAKE + 2), -1), (dict(y=FAKE + 1), -1),
    (dict(T=1 << 20, H=64, D=64), -2),  # a slice beyond 2^31 bytes of offsets
    (dict(B=1 << 16, H=1 << 16), -2),   # grid beyond one launch
])
def test_recurrence_rejects_invalid(lib, kw, status):
    assert rec(lib, **kw) == status


def test_recurrence_flops():
    assert osa.attn_gated_recurrence_flops(2, 128, 4, 24) == 5 * 2 * 128 * 4 * 24 * 24
    assert osa.attn_gated_recurrence_flops(0, 1, 1, 1) == 0.0


def test_decode_workspace_bytes():
    for B, H, Tq, Tk in [(1, 1, 1, 1), (4, 12, 1, 8192), (2, 3, 33, 1000)]:
        sizes = {}
        for D in (32, 64, 128):
            n = osa.attn_decode_workspace_bytes(B, H, Tq, Tk, D)
            assert n > 0 and n % 256 == 0
            # at least one partial (D floats + lse) per row
            assert n >= B * H * Tq * (D + 1) * 4
            sizes[D] = n
        assert sizes[32] <= sizes[64] <= sizes[128]
        assert osa.attn_decode_workspace_bytes(B, H, Tq, Tk) == sizes[64]
    assert osa.attn_decode_workspace_bytes(1, 1, 5, 4) == 0
    assert osa.attn_decode_workspace_bytes(0, 1, 1, 1) == 0
    for D in (16, 48, 96, 256):
        assert osa.attn_decode_workspace_bytes(1, 1, 1, 8, D) == 0


def test_naive_workspace_bytes():
    for B, H, T in [(1, 1, 256), (1, 1, 4096), (2, 3, 1000), (1, 1, 1)]:
        want = (2 * B * H * T * T + B * H * T) * 4
        want = (want + 255) // 256 * 256
        assert osa.attn_naive_workspace_bytes(B, H, T) == want
    assert osa.attn_naive_workspace_bytes(0, 1, 1) == 0
    assert osa.attn_naive_workspace_bytes(1 << 30, 1 << 30, 1 << 30) == 0


def test_flops_convention():
    g = GOLDEN["causal_fwd_rate"]
    fl = osa.attn_flops(g["B"], g["H"], g["T"], g["D"], True)
    assert fl == 2.0 * g["B"] * g["H"] * g["T"] ** 2 * g["D"]
    assert osa.attn_flops(1, 1, 10, 64, False) == 4 * 100 * 64
    for ms, tflops in g["cases"]:
        assert abs(fl / (ms * 1e-3) / 1e12 - tflops) <= g["rate_tolerance_tflops"]
    assert osa.attn_flops(0, 1, 1, 64, True) == 0.0


def test_naive_traffic_matches_pages():
    per_head = GOLDEN["score_table_bytes_per_head_fp32"]["cases"]
    passes = GOLDEN["naive_passes_over_table"]["passes"]
    for n, table in per_head:
        t = osa.attn_traffic_bytes(osa.ATTN_PATH_NAIVE, 1, 1, n, 64,
                                   osa.ATTN_F32, False)
        assert t["score_matrix"] == passes * table
        assert t["table_bytes"] >= 2 * table
        assert t["floor"] == 4 * n * 64 * 4 + 4 * n
        assert t["ask"] > t["score_matrix"]
    for T, approx, rel in GOLDEN["score_entries_per_head"]["cases"]:
        t = osa.attn_traffic_bytes(osa.ATTN_PATH_NAIVE, 1, 1, T, 64,
                                   osa.ATTN_F32, True)
        entries = t["score_matrix"] / (passes * 4)
        assert abs(entries - approx) / approx <= rel
    g = GOLDEN["eval_table_bytes"]
    t = osa.attn_traffic_bytes(osa.ATTN_PATH_NAIVE, g["B"], g["H"], g["T"], 64,
                               osa.ATTN_F32, True)
    assert round(t["score_matrix"] / passes / 2 ** 30, 1) == g["gib"]


def fused_ask_closed_form(B, H, T, dtype, causal):
    """K and V rows fetched per query tile, summed: written out directly from
    the tile sizes rather than through the library's loop."""
    bm, bn = osa.attn_fused_tile(dtype)
    if dtype == osa.ATTN_F32 and -(-T // 128) * B * H < 256:
        bm = 32  # the key-split kernel's 32-row tiles on small grids
    if dtype != osa.ATTN_F32 and -(-T // 256) * B * H >= 256:
        bm = 256  # the eight-wave kernel's 256-row tiles on large grids
    elt = 4 if dtype == osa.ATTN_F32 else 2
    nq = -(-T // bm)
    rows = 0
    for qt in range(nq):
        last = min(T - 1, qt * bm + bm - 1) if causal else T - 1
        rows += min(T, (last // bn + 1) * bn)
    tensor = B * H * T * 64 * elt
    return 2 * tensor + 4 * B * H * T + 2 * B * H * rows * 64 * elt


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 100, 256, 1000, 8192])
def test_fused_traffic(dtype, causal, T):
    t = osa.attn_traffic_bytes(osa.ATTN_PATH_FUSED, 4, 12, T, 64, dtype, causal)
    elt = 4 if dtype == 0 else 2
    assert t["floor"] == 4 * 4 * 12 * T * 64 * elt + 4 * 4 * 12 * T
    assert t["score_matrix"] == 0 and t["table_bytes"] == 0
    assert t["ask"] == fused_ask_closed_form(4, 12, T, dtype, causal)
    assert t["ask"] >= t["floor"]


def test_fused_kernel_selection():
    """attn_fused_kernel names the kernel attn_fwd launches. 16-bit, D = 64:
    the eight-wave kernel on full calls once its 256-row grid reaches 256
    workgroups and on causal calls once B*H*(ceil(T/256) + 1) >= 600; its
    key-split form on the other causal calls and on full calls of at most
    256 128-row workgroups; the 128-row kernel on the full calls between.
    Then the fp32 key-split kernel on small fp32 grids and the head-dim
    kernels for D = 32 / 128; invalid arguments give attn_fwd's status."""
    name = lambda *a: osa.attn_kernel_name(osa.attn_fused_kernel(*a))
    assert name(4, 12, 8192, 64, True, osa.ATTN_BF16) == "fused_fwd16w8<bf16, causal>"   # 1584
    assert name(4, 12, 8192, 64, False, osa.ATTN_F16) == "fused_fwd16w8<f16, full>"
    assert name(4, 12, 4096, 64, True, osa.ATTN_BF16) == "fused_fwd16w8<bf16, causal>"   # 816
    assert name(8, 16, 1024, 64, True, osa.ATTN_BF16) == "fused_fwd16w8<bf16, causal>"   # 640
    assert name(2, 16, 4096, 64, True, osa.ATTN_BF16) == "fused_fwd16w8s<bf16, causal>"  # 544
    assert name(4, 12, 2048, 64, True, osa.ATTN_BF16) == "fused_fwd16w8s<bf16, causal>"  # 432
    assert name(4, 12, 1024, 64, True, osa.ATTN_F16) == "fused_fwd16w8s<f16, causal>"    # 240
    assert name(4, 12, 2048, 64, False, osa.ATTN_BF16) == "fused_fwd16w8<bf16, full>"    # 384
    assert name(1, 256, 1, 64, False, osa.ATTN_F16) == "fused_fwd16w8<f16, full>"        # 256
    assert name(4, 12, 1024, 64, False, osa.ATTN_BF16) == "fused_fwd16<bf16, full>"      # 384 rows/128
    assert name(1, 255, 1, 64, False, osa.ATTN_F16) == "fused_fwd16w8s<f16, full>"       # 255 rows/128
    assert name(1, 1, 300, 64, False, osa.ATTN_BF16) == "fused_fwd16w8s<bf16, full>"
    assert name(1, 1, 4096, 64, False, osa.ATTN_F32) == "fused_fwd32_split<full>"
    assert name(8, 64, 4096, 64, True, osa.ATTN_F32) == "fused_fwd32<causal>"
    assert name(4, 12, 8192, 128, True, osa.ATTN_BF16) == "fused_hd16<bf16, causal, 128>"
    assert name(4, 12, 8192, 32, False, osa.ATTN_F16) == "fused_hd16<f16, full, 32>"
    lib = binding.load()
    assert lib.attn_fused_kernel(0, 1, 8, 64, 1, 1) == -1
    assert lib.attn_fused_kernel(1, 1, 8, 64, 1, 7) == -1
    assert lib.attn_fused_kernel(1, 1, 8, 48, 1, 1) == -2
    assert lib.attn_fused_kernel(1, 1, 8, 128, 1, 0) == -2


def test_metric_workload_floor():
    """Q, K, V, O once in bf16 plus the fp32 lse at 4 x 12 x 8192 x 64."""
    t = osa.attn_traffic_bytes(osa.ATTN_PATH_FUSED, 4, 12, 8192, 64,
                               osa.ATTN_BF16, True)
    assert t["floor"] == 4 * 50331648 + 1572864 == 202899456


def test_traffic_rejects_invalid(lib):
    assert lib.attn_traffic_bytes(0, 1, 1, 8, 64, 1, 1, None) == -1
    out = binding.attn_traffic()
    import ctypes
    assert lib.attn_traffic_bytes(2, 1, 1, 8, 64, 1, 1, ctypes.byref(out)) == -1
    assert lib.attn_traffic_bytes(1, 1, 1, 8, 64, 1, 1, ctypes.byref(out)) == -2
    assert lib.attn_traffic_bytes(0, 1, 1, 8, 63, 1, 1, ctypes.byref(out)) == -2
    # head dims 32 and 128: the 16-bit fused path only
    assert lib.attn_traffic_bytes(0, 1, 1, 8, 128, 1, 1, ctypes.byref(out)) == 0
    assert lib.attn_traffic_bytes(0, 1, 1, 8, 32, 2, 1, ctypes.byref(out)) == 0
    assert lib.attn_traffic_bytes(0, 1, 1, 8, 32, 0, 1, ctypes.byref(out)) == -2
    assert lib.attn_traffic_bytes(1, 1, 1, 8, 128, 0, 1, ctypes.byref(out)) == -2


@pytest.mark.parametrize("D", [32, 128])
def test_traffic_other_head_dims(D):
    """The fused ask for D = 32 / 128 counts the same 64-key tiles as D = 64,
    with rows of 2 D bytes: everything scales with D."""
    a = osa.attn_traffic_bytes(0, 2, 3, 1000, D, 1, True)
    b = osa.attn_traffic_bytes(0, 2, 3, 1000, 64, 1, True)
    lse_bytes = 2 * 3 * 1000 * 4
    for key in ("floor", "ask"):
        assert (a[key] - lse_bytes) * 64 == (b[key] - lse_bytes) * D


def test_kernel_table(lib):
    n = osa.attn_kernel_count()
    assert n == 91
    names = [osa.attn_kernel_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert osa.attn_kernel_name(n) is None
    assert lib.attn_kernel_attributes(n, None) == -1
    assert lib.attn_kernel_attributes(0, None) == -1


def test_binding_without_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.load(str(tmp_path / "missing.so"))
