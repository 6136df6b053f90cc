#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the fused forward (attn_fwd_stream) over the metric's
workload: causal, head dim 64, bf16 in / fp32 accumulate, B = 4 sequences x
H = 12 heads x T = 8192 tokens, seeded N(0,1) inputs already resident in HBM
("Flash attention in PyTorch, then in Triton" measures this shape on its
RTX 4090, section "A kernel in Triton"). The FLOP count is the pages'
convention, 2*B*H*T^2*D for causal attention (section "Attention by hand").

Order of work, as the page "attention.cu" does it: the traffic arithmetic of
both paths is printed first (stderr), then the output is checked against the
double oracle on a seeded row sample (which is also the timed CPU baseline),
and only then is anything timed. One JSON line goes to stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

# The oracle's OpenMP threads go to sleep once a CPU leg ends instead of
# spinning, so they do not take the host cores that launch the timed GPU
# work (a spinning pool delayed a launch inside an event pair by tens of
# milliseconds). Must be set before the OpenMP runtime starts.
os.environ.setdefault("OMP_WAIT_POLICY", "PASSIVE")

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attention fwd TFLOP/s (causal, d=64, bf16, T=8192) and % of MFMA "
          "peak")
# MI355X published dense peaks
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
BF16_TOL, F32_TOL_BASE = 2e-2, 1e-5
TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                            "fused_bf16_causal_b4h12_t8192_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "online_softmax_amd", "csrc", f)
                  for f in ("fused_fwd.hip", "fused_layout.h", "gfx950.h", "online_step.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM-side bytes per launch from the committed PMC summary, if it was
    taken on the kernel source as it is now; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fmt_bytes(n):
    return f"{n:>16,d} B  ({n / 2**20:10.2f} MiB)"


def print_traffic(osa, w):
    """Bytes before any time (the fused path, and the naive path's table
    cost at this shape in fp32, which is the contrast)."""
    dt = {"f32": osa.ATTN_F32, "bf16": osa.ATTN_BF16, "f16": osa.ATTN_F16}[w.dtype]
    f = osa.attn_traffic_bytes(osa.ATTN_PATH_FUSED, w.B, w.H, w.T, w.D, dt,
                               w.causal)
    n = osa.attn_traffic_bytes(osa.ATTN_PATH_NAIVE, w.B, w.H, w.T, w.D,
                               osa.ATTN_F32, w.causal)
    log(f"traffic arithmetic, {w.name} (before any timing):")
    log(f"  fused floor (Q,K,V,O once + lse) {fmt_bytes(f['floor'])}")
    log(f"  fused ask (K,V per query tile)   {fmt_bytes(f['ask'])}")
    log(f"  naive score-table passes (fp32)  {fmt_bytes(n['score_matrix'])}")
    log(f"  naive table memory (fp32)        {fmt_bytes(n['table_bytes'])}")
    log(f"  naive / fused floor traffic      {(n['score_matrix'] + n['floor']) / n['floor']:.1f}x")
    return f, n


def print_kernel_table(osa):
    log(f"  {'kernel':28s} {'regs':>5s} {'LDS B':>7s} {'spill B':>8s} {'WG/CU':>6s}")
    rows = {}
    for i in range(osa.attn_kernel_count()):
        a = osa.attn_kernel_attributes(i)
        name = osa.attn_kernel_name(i)
        rows[name] = a
        log(f"  {name:28s} {a['num_regs']:5d} {a['lds_bytes']:7d} "
            f"{a['private_bytes']:8d} {a['workgroups_per_cu']:6d}")
    return rows


def cpu_baseline(oracle, q, k, v, o, lse, w, nrows, seed):
    """The double oracle, as it stands, on a seeded row sample of the same
    workload: its rate (scaled to TFLOP/s by the rows' own visible keys) and
    the GPU output's error on those rows."""
    import numpy as np
    from online_softmax_amd.inputs import sample_rows
    rows = sample_rows(w.B, w.H, w.T, nrows, seed)
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    ro, rl = oracle.attention(qn, kn, vn, w.causal, w.scale, rows=rows,
                              threads=threads)
    dt = time.perf_counter() - t0
    t = rows % w.T
    visible = (t + 1) if w.causal else np.full_like(t, w.T)
    flops = float((4 * w.D * visible).sum())
    got_o = o.reshape(-1, w.D).float().cpu().numpy()[rows]
    got_l = lse.reshape(-1).cpu().numpy()[rows]
    err_o = float(np.abs(got_o.astype(np.float64) - ro).max())
    err_l = float(np.abs(got_l.astype(np.float64) - rl).max())
    finite = bool(np.isfinite(got_o).all() and np.isfinite(got_l).all())
    full = 2.0 * w.B * w.H * w.T * w.T * w.D * (1 if w.causal else 2)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(rows)} seeded rows (of {w.rows}) of {w.name}, all "
                   f"{w.D} dims, {flops:.3e} flop in {dt:.2f} s on {threads} "
                   f"threads of {cpu_model()}"),
        "extrapolated_full_s": full / (flops / dt),
    }, {"rows": int(len(rows)), "max_abs_err_o": err_o,
        "max_abs_err_lse": err_l, "finite": finite}


def oracle_single_core(oracle):
    """The double oracle on one core for the page "attention.cu"'s one-head
    case (256 tokens) and the largest of the two-sequence, three-head causal
    cases (1000 tokens), whole, as that page times its CPU reference on one
    core: seconds and GFLOP/s (4 D flop per visible query-key pair)."""
    from online_softmax_amd.inputs import WORKLOADS, workload_qkv
    out = []
    for name in ("single_head_n256_f32", "causal_b2h3_t1000_f32"):
        w = WORKLOADS[name]
        q, k, v = (x.float().numpy() for x in workload_qkv(w))
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.causal, w.scale, threads=1)
        dt = time.perf_counter() - t0
        pairs = w.B * w.H * (w.T * (w.T + 1) // 2 if w.causal else w.T * w.T)
        flops = 4.0 * w.D * pairs
        out.append({"workload": name, "seconds": dt, "flop": flops,
                    "gflops": flops / dt / 1e9, "cores": 1})
        log(f"oracle on one core, {name}: {dt:.3f} s, {flops / dt / 1e9:.2f} GFLOP/s")
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def timed_calls(torch, run, stream, steps, warmup=5):
    """A leg's timing: the time-based warm-up, then `steps` calls timed by
    time_steps (mean launch duration from the bracketing event pair, the
    per-call median and min, and how many calls paused on the device)."""
    calls, _ = warm_up(torch, run, stream, warmup)
    r = time_steps(torch, run, stream, steps)
    r["warmup_calls"] = calls
    return r


def warm_up(torch, run, stream, min_calls, min_ms=300.0, batch=10):
    """Launch run() until at least `min_calls` calls and at least `min_ms` of
    device time have gone by (HIP events around each batch): clocks and caches
    settle before anything is timed, whatever the call count asked for.
    Returns (calls, device ms)."""
    calls, spent = 0, 0.0
    while calls < min_calls or spent < min_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(batch):
            run()
        b.record(stream)
        b.synchronize()
        calls += batch
        spent += a.elapsed_time(b)
        if calls >= 100000:
            break
    torch.cuda.synchronize()
    return calls, spent


def time_steps(torch, run, stream, steps):
    """K calls issued back to back and timed as one region bracketed by
    synchronisation (wall clock: the step time) and by one HIP event pair on
    the launch stream (its span over K: the mean launch duration). Then a
    second round of K calls, each bracketed by an event pair of its own, for
    the per-call median, min and max: calls whose device time exceeds twice
    the median are counted as device-side pauses. The second round is kept
    out of the timed region because an event pair around every call puts
    host work and timestamp packets between the launches (0.43 against 0.42
    ms per call at the metric workload, and at 20-microsecond calls the GPU
    then waits on the host). Wall time beyond the first round's event span
    is host-side time."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    span = e0.elapsed_time(e1)
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    med = statistics.median(per)
    slow = [x for x in per if x > 2.0 * med]
    return {"wall_ms_per_step": wall / steps, "mean": span / steps, "median": med,
            "min": min(per), "max": max(per), "per_call_mean": statistics.fmean(per),
            "per_call": [round(x, 4) for x in per],
            "device_pauses": len(slow), "device_pause_ms": sum(slow) - med * len(slow),
            "host_ms": max(0.0, wall - span)}


def backward_leg(osa, torch, oracle, w, q, k, v, qd, kd, vd, o, lse, steps=20,
                 warmup=3, with_oracle=True, atomic=False, cache=None):
    """The backward pass (attn_bwd_stream, or with atomic=True
    attn_bwd_atomic_stream) on the same workload for a seeded output
    gradient: a correctness gate against the double oracle on one whole
    slice (also the backward's CPU baseline; `cache` keeps the oracle's
    gradients for the second leg), then HIP-event timing. Throughput uses
    the pages' count for the pass, five products to the forward's two
    ("Flash attention in PyTorch, then in Triton", section "Backwards, and
    training with it"); the two-kernel split performs seven, the atomic
    path five."""
    import numpy as np
    from online_softmax_amd.inputs import make_qkv
    dev = qd.device
    (dout,) = make_qkv(w.B, w.H, w.T, w.D, w.dtype, w.seed + 7)[:1]
    dd = dout.to(dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = (osa.attn_bwd_atomic_workspace_bytes if atomic else osa.attn_bwd_workspace_bytes)
    ws = torch.empty(need(w.B, w.H, w.T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    entry = osa.attn_bwd_atomic_stream if atomic else osa.attn_bwd_stream
    run = lambda: entry(qd, kd, vd, o, dd, lse, dq, dk, dv, ws, w.causal, w.scale, stream)
    run()
    torch.cuda.synchronize()
    out = {"entry": "attn_bwd_atomic_stream" if atomic else "attn_bwd_stream",
           "kernels": (["bwd_prep16", "bwd_kvq16", "bwd_dq_finish16"] if atomic
                       else ["bwd_delta16", "bwd_kv16", "bwd_q16"])}
    flops = osa.attn_bwd_flops(w.B, w.H, w.T, w.D, w.causal)
    performed = 5.0 if atomic else 7.0
    if with_oracle:
        sl = np.array([0])
        threads = oracle.max_threads()
        cache = {} if cache is None else cache
        t0 = time.perf_counter()
        if "want" not in cache:
            cache["want"] = oracle.attention_backward(q, k, v, dout, w.causal, w.scale,
                                                      slices=sl, threads=threads)
            cache["dt"] = time.perf_counter() - t0
        want, dt = cache["want"], cache["dt"]
        errs, ok = {}, True
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
            got = g.float().cpu().numpy().reshape(w.B * w.H, w.T, w.D)[sl]
            bound = 2e-2 * max(1.0, float(np.abs(ref).max()))
            e = float(np.abs(got - ref).max())
            fin = bool(np.isfinite(got).all())
            errs[name] = {"max_abs_err": e, "bound": bound, "finite": fin}
            ok = ok and fin and e <= bound
        out["parity"] = {"slices": sl.tolist(), "grads": errs, "pass": ok}
        slice_flops = flops / (w.B * w.H)
        out["cpu_baseline"] = {
            "value": slice_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"gradients of slice 0 (of {w.B * w.H}) of {w.name}, "
                       f"{slice_flops:.3e} flop by the pages' count in {dt:.2f} s "
                       f"on {threads} threads of {cpu_model()}")}
        log(f"backward ({out['entry']}) parity on slice 0: {errs}")
        if not ok:
            log("backward correctness gate FAILED: not timing it")
            out["pass"] = False
            return out
    ms = timed_calls(torch, run, stream, steps, warmup)
    mean = ms["mean"]
    achieved = flops / (mean * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    out.update({
        "ms": ms,
        "flop_convention": flops, "flop_performed": flops * performed / 5.0,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "achieved_performed": achieved * performed / 5.0},
        "pass": True})
    log(f"backward ({out['entry']}): mean {mean:.4f} ms, {achieved:.1f} TFLOP/s by the "
        f"pages' count ({achieved * performed / 5.0:.1f} performed) = "
        f"{100 * achieved / peak:.1f}% of {peak}")
    del dq, dk, dv, ws, dd
    return out


def decode_leg(osa, torch, oracle, B=4, H=12, Tq=1, Tk=8192, D=64, dtype="bf16", steps=20,
               copies=4, with_oracle=True):
    """The decode path (attn_decode_stream): Tq new tokens per sequence
    against a Tk-token key/value cache, causal. It reads the cache once, so
    it is bound by HBM: the figure is algorithmic bytes (K and V once, q and o
    once) per call over the call's time, against 8 TB/s. Timed calls rotate
    over `copies` caches, together larger than the 256 MB Infinity Cache, so
    the reads reach HBM. A correctness gate against the double oracle on
    every row comes first (also this leg's CPU baseline)."""
    import numpy as np
    from online_softmax_amd.inputs import make_qkv
    dev = torch.device("cuda:0")
    scale = 0.125
    seed = 2101 if D == 64 else 2111
    (q,) = make_qkv(B, H, Tq, D, dtype, seed)[:1]
    caches = [make_qkv(B, H, Tk, D, dtype, seed + 1 + i)[1:] for i in range(copies)]
    qd = q.to(dev)
    kv = [(k.to(dev), v.to(dev)) for k, v in caches]
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    ws = torch.empty(osa.attn_decode_workspace_bytes(B, H, Tq, Tk, D), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    dname = "" if D == 64 else f"_d{D}"
    out = {"workload": f"decode_b{B}h{H}_tq{Tq}_tk{Tk}{dname}_{dtype}", "B": B, "H": H,
           "Tq": Tq, "Tk": Tk, "D": D, "causal": True, "scale": scale,
           "kernels": ["decode_split16", "decode_combine16"]}
    osa.attn_decode_stream(qd, kv[0][0], kv[0][1], o, lse, ws, True, scale, stream)
    torch.cuda.synchronize()
    if with_oracle:
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        ro, rl = oracle.attention_kv(q, caches[0][0], caches[0][1], True, scale,
                                     threads=threads)
        dt = time.perf_counter() - t0
        eo = float(np.abs(o.float().cpu().numpy() - ro).max())
        el = float(np.abs(lse.cpu().numpy() - rl).max())
        ok = eo <= BF16_TOL and el <= BF16_TOL and bool(torch.isfinite(o.float()).all())
        out["parity"] = {"rows": B * H * Tq, "max_abs_err_o": eo, "max_abs_err_lse": el,
                         "bound": BF16_TOL, "pass": ok}
        kv_bytes = 2 * B * H * Tk * D * (4 if dtype == "f32" else 2)
        out["cpu_baseline"] = {
            "value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"every row of the decode workload in {dt:.2f} s on {threads} "
                      f"threads of {cpu_model()}"}
        log(f"decode parity: {out['parity']}")
        if not ok:
            log("decode correctness gate FAILED: not timing it")
            out["pass"] = False
            return out
    for i in range(3 * copies):
        k, v = kv[i % copies]
        osa.attn_decode_stream(qd, k, v, o, lse, ws, True, scale, stream)
    torch.cuda.synchronize()

    def rotating(entry, *outs):
        # each call reads the next cache, so consecutive calls share no bytes
        n = [0]

        def call():
            k, v = kv[n[0] % copies]
            n[0] += 1
            entry(qd, k, v, *outs)
        return call

    # calls back to back (the call's time in a decode loop), then a round
    # with an event pair per call for the median
    r = time_steps(torch, rotating(lambda *x: osa.attn_decode_stream(*x, ws, True, scale, stream),
                                   o, lse), stream, steps)
    mean, med = r["mean"], r["median"]
    elt = 2
    algo = 2 * B * H * Tk * D * elt + 2 * B * H * Tq * D * elt + 4 * B * H * Tq
    achieved = algo / (mean * 1e-3) / 1e9
    out.update({"ms": {"back_to_back": mean, "median": med, "per_call_mean": r["per_call_mean"],
                       "min": r["min"]},
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                             "algorithmic_bytes_per_call": algo},
                "pass": True})
    log(f"decode D={D}: {mean * 1e3:.1f} us per call back to back (per-call median "
        f"{med * 1e3:.1f}), {achieved:.0f} GB/s = {100 * achieved / PEAK_HBM_GBS:.1f}% of "
        f"{PEAK_HBM_GBS:.0f} GB/s")
    # the same calls from a HIP graph (a serving loop without per-launch host
    # work): `copies` calls, one per cache, captured once and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for k, v in kv:
            osa.attn_decode_stream(qd, k, v, o, lse, ws, True, scale)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for k, v in kv:
            osa.attn_decode_stream(qd, k, v, o, lse, ws, True, scale)
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    rg = time_steps(torch, graph.replay, stream, reps)
    g_us = rg["mean"] / copies * 1e3
    out["graph_replay_us_per_call"] = g_us
    out["graph_replay_GBs"] = algo / (g_us * 1e-6) / 1e9
    log(f"decode D={D} from a HIP graph: {g_us:.1f} us per call, "
        f"{algo / (g_us * 1e-6) / 1e9:.0f} GB/s")
    del graph
    # the same calls through the entry point that allocates nothing (one
    # launch: the last workgroup of each tile merges the split partials),
    # checked against the workspace entry point's output first
    o2 = torch.empty_like(qd)
    lse2 = torch.empty_like(lse)
    osa.attn_decode_stream(qd, kv[0][0], kv[0][1], o, lse, ws, True, scale, stream)
    osa.attn_decode_noalloc_stream(qd, kv[0][0], kv[0][1], o2, lse2, True, scale, stream)
    torch.cuda.synchronize()
    d_o = float((o2.float() - o.float()).abs().max())
    d_l = float((lse2 - lse).abs().max())
    na = {"entry": "attn_decode_noalloc_stream", "kernels": ["decode_merged16"],
          "vs_workspace_entry": {"max_abs_d_o": d_o, "max_abs_d_lse": d_l},
          "pass": d_o <= BF16_TOL and d_l <= BF16_TOL}
    if na["pass"]:
        for i in range(3 * copies):
            k, v = kv[i % copies]
            osa.attn_decode_noalloc_stream(qd, k, v, o2, lse2, True, scale, stream)
        torch.cuda.synchronize()
        r2 = time_steps(torch, rotating(
            lambda *x: osa.attn_decode_noalloc_stream(*x, True, scale, stream), o2, lse2),
            stream, steps)
        mean2 = r2["mean"]
        ach2 = algo / (mean2 * 1e-3) / 1e9
        na.update({"ms": {"back_to_back": mean2, "median": r2["median"],
                          "per_call_mean": r2["per_call_mean"], "min": r2["min"]},
                   "roofline": {"bound": "hbm", "achieved": ach2, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": ach2 / PEAK_HBM_GBS}})
        log(f"decode D={D} without allocation (one launch): {mean2 * 1e3:.1f} us per call back "
            f"to back (median {r2['median'] * 1e3:.1f}), {ach2:.0f} GB/s = "
            f"{100 * ach2 / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f} GB/s")
    else:
        log(f"decode D={D} without allocation: differs from the workspace entry point "
            f"({d_o:.3e}, {d_l:.3e}); not timed")
    out["noalloc"] = na
    del o2, lse2
    del kv, qd, o, lse, ws
    return out


def head_dim_leg(osa, torch, oracle, D, B=4, H=12, T=8192, dtype="bf16", steps=10,
                 with_oracle=True, gate_rows=512):
    """The fused forward at another head dimension (32 or 128) on the same
    4 x 12 x 8192 causal shape: a correctness gate against the double oracle
    on sampled rows, then HIP-event timing. Bound by the matrix cores like
    D = 64: 4 T^2 D flop per slice, halved by the causal mask."""
    import numpy as np
    from online_softmax_amd.inputs import make_qkv, sample_rows
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    q, k, v = make_qkv(B, H, T, D, dtype, 2200 + D)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    run = lambda: osa.attn_fwd_stream(qd, kd, vd, o, lse, True, scale, stream)
    run()
    torch.cuda.synchronize()
    out = {"workload": f"b{B}h{H}_t{T}_d{D}_{dtype}_causal", "B": B, "H": H, "T": T,
           "D": D, "scale": scale, "kernels": [f"fused_hd16<{dtype}, causal, {D}>"]}
    flops = osa.attn_flops(B, H, T, D, True)
    if with_oracle:
        rows = sample_rows(B, H, T, gate_rows, 2300 + D, boundaries=(64, 128, T // 2))
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        ro, rl = oracle.attention(q, k, v, True, scale, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        eo = float(np.abs(o.float().cpu().numpy().reshape(-1, D)[rows] - ro).max())
        el = float(np.abs(lse.cpu().numpy().reshape(-1)[rows] - rl).max())
        ok = eo <= BF16_TOL and el <= BF16_TOL and bool(torch.isfinite(o.float()).all())
        out["parity"] = {"rows": int(len(rows)), "max_abs_err_o": eo, "max_abs_err_lse": el,
                         "bound": BF16_TOL, "pass": ok}
        row_flops = flops / (B * H * T)
        out["cpu_baseline"] = {
            "value": row_flops * len(rows) / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(rows)} sampled rows (mean causal row cost) in {dt:.2f} s on "
                      f"{threads} threads of {cpu_model()}"}
        log(f"D={D} parity: {out['parity']}")
        if not ok:
            log(f"D={D} correctness gate FAILED: not timing it")
            out["pass"] = False
            return out
    ms = timed_calls(torch, run, stream, steps)
    mean = ms["mean"]
    achieved = flops / (mean * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    out.update({"ms": ms,
                "flop_per_call": flops,
                "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                             "unit": "TFLOP/s", "frac": achieved / peak},
                "pass": True})
    log(f"D={D}: mean {mean:.4f} ms, {achieved:.1f} TFLOP/s = "
        f"{100 * achieved / peak:.1f}% of {peak}")
    del qd, kd, vd, o, lse
    return out


# The float32 FMA rate one VALU instruction per lane reaches (half the
# published 157.3 TFLOP/s vector peak, which counts packed two-wide FMAs;
# this library is compiled without packed fp32 instructions).
PEAK_FP32_FMA_TFLOPS = 78.6


def recurrence_leg(osa, torch, oracle, with_oracle=True, steps=20):
    """The gated linear recurrence (attn_gated_recurrence_stream, float32)
    at two sizes: the page's own 2 x 128 x 4 x 24 [B, T, H, D], which one
    sequential pass per column bounds by latency (the figure is the call's
    median time), and 8 x 4096 x 32 x 64, which has work for every SIMD and
    is bound by vector arithmetic (5 B T H D^2 flop against the fp32 vector
    peak). Each size passes a correctness gate against the double oracle
    first; the page-size gate is also the CPU baseline."""
    import numpy as np
    from online_softmax_amd.inputs import make_gated
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {"kernels": ["gated_recurrence32"]}

    def bound_ok(y, q, k, v, g):
        want = oracle.gated_recurrence(q, k, v, g)
        mag = oracle.gated_recurrence(q.abs(), k.abs(), v.abs(), g)
        t = np.arange(q.shape[1], dtype=np.float64).reshape(1, -1, 1, 1)
        bound = 2.0 * (q.shape[3] + t + 2) * 2.0 ** -24 * mag + 1e-30
        ratio = float((np.abs(y - want) / bound).max())
        return ratio, bool(np.isfinite(y).all()) and ratio <= 1.0

    for label, (B, T, H, D), seed in (("page", (2, 128, 4, 24), 2401),
                                      ("throughput", (8, 4096, 32, 64), 2402)):
        q, k, v, g = make_gated(B, T, H, D, seed)
        args = [x.to(dev) for x in (q, k, v, g)]
        y = torch.empty_like(args[0])
        osa.attn_gated_recurrence_stream(*args, y, stream)
        torch.cuda.synchronize()
        rec = {"B": B, "T": T, "H": H, "D": D}
        if with_oracle:
            yh = y.cpu().numpy()
            if label == "page":
                threads = oracle.max_threads()
                t0 = time.perf_counter()
                reps = 0
                while reps < 20 or time.perf_counter() - t0 < 0.5:
                    oracle.gated_recurrence(q, k, v, g, threads=threads)
                    reps += 1
                dt = (time.perf_counter() - t0) / reps
                ratio, ok = bound_ok(yh, q, k, v, g)
                rec["cpu_baseline"] = {
                    "value": osa.attn_gated_recurrence_flops(B, T, H, D) / dt / 1e9,
                    "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
                    "sample": f"the whole page-size call, {dt * 1e3:.3f} ms per call "
                              f"({reps} calls) on {threads} threads of {cpu_model()}"}
            else:
                sl = [x[:1, :, :1].contiguous() for x in (q, k, v, g)]
                ratio, ok = bound_ok(yh[:1, :, :1], *sl)
            rec["parity"] = {"max_err_over_bound": ratio, "pass": ok,
                             "checked": "every element" if label == "page" else
                             "slice (b=0, h=0)"}
            log(f"recurrence {label} parity: {rec['parity']}")
            if not ok:
                log(f"recurrence {label} correctness gate FAILED: not timing it")
                rec["pass"] = False
                out[label] = rec
                continue
        ms = timed_calls(torch, lambda: osa.attn_gated_recurrence_stream(*args, y, stream),
                         stream, steps)
        # the page-size call lasts less than the host's own time per call, so
        # calls do not queue up: its figure is the median of single calls;
        # the large size queues and takes the bracketed mean
        med = ms["median"] if label == "page" else ms["mean"]
        flops = osa.attn_gated_recurrence_flops(B, T, H, D)
        rec["ms"] = ms
        rec["flop_per_call"] = flops
        achieved = flops / (med * 1e-3) / 1e12
        rec["roofline"] = {"bound": "latency" if label == "page" else "alu",
                           "achieved": achieved, "peak": PEAK_FP32_FMA_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_FMA_TFLOPS}
        rec["pass"] = True
        log(f"recurrence {label} {B}x{T}x{H}x{D}: {med * 1e3:.1f} us per call, "
            f"{achieved:.2f} TFLOP/s ({100 * achieved / PEAK_FP32_FMA_TFLOPS:.1f}% of "
            f"the one-issue fp32 FMA rate)")
        out[label] = rec
        del args, y
    return out


def contrast(osa, torch, oracle, steps=10):
    """Both paths on the fp32 single-head workloads of the page
    "attention.cu" (bytes first, then a correctness gate, then time)."""
    from online_softmax_amd.inputs import WORKLOADS, workload_qkv
    import numpy as np
    out = []
    for name in ("single_head_n1024_f32", "single_head_n4096_f32"):
        w = WORKLOADS[name]
        f = osa.attn_traffic_bytes(osa.ATTN_PATH_FUSED, 1, 1, w.T, 64,
                                   osa.ATTN_F32, False)
        n = osa.attn_traffic_bytes(osa.ATTN_PATH_NAIVE, 1, 1, w.T, 64,
                                   osa.ATTN_F32, False)
        log(f"{name}: naive score-table traffic {n['score_matrix']:,d} B, "
            f"fused floor {f['floor']:,d} B, fused ask {f['ask']:,d} B")
        q, k, v = (x.cuda() for x in workload_qkv(w))
        o_f, o_n = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((1, 1, w.T), device=q.device)
        ws = torch.empty(osa.attn_naive_workspace_bytes(1, 1, w.T),
                         dtype=torch.uint8, device=q.device)
        osa.attn_fwd_stream(q, k, v, o_f, lse, False, w.scale)
        osa.attn_naive_fwd(q, k, v, o_n, None, ws, False, w.scale)
        torch.cuda.synchronize()
        ro, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu(), False, w.scale)
        bound = max(F32_TOL_BASE, F32_TOL_BASE * math.sqrt(w.T / 256))
        ef = float(np.abs(o_f.cpu().numpy() - ro).max())
        en = float(np.abs(o_n.cpu().numpy() - ro).max())

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        ms_f = timed(lambda: osa.attn_fwd_stream(q, k, v, o_f, lse, False,
                                                 w.scale))
        ms_n = timed(lambda: osa.attn_naive_fwd(q, k, v, o_n, None, ws, False,
                                                w.scale))
        fl = osa.attn_flops(1, 1, w.T, 64, False)
        row = {"workload": name, "fused_ms": ms_f, "naive_ms": ms_n,
               "fused_tflops": fl / ms_f / 1e9, "naive_tflops": fl / ms_n / 1e9,
               "naive_table_traffic_B": n["score_matrix"],
               "fused_floor_B": f["floor"], "fused_ask_B": f["ask"],
               "max_abs_err_fused": ef, "max_abs_err_naive": en,
               "bound": bound, "pass": ef <= bound and en <= bound}
        log(f"  fused {ms_f:.4f} ms (err {ef:.2e}), naive {ms_n:.4f} ms "
            f"(err {en:.2e}), naive/fused time {ms_n / ms_f:.1f}x")
        out.append(row)
        del q, k, v, o_f, o_n, ws
    return out


def forward_case(osa, torch, oracle, B, H, T, dtype, seed, steps, warmup,
                 gate_rows=256, label=None):
    """One fused-forward case other than the headline: seeded inputs, a
    correctness gate against the double oracle on `gate_rows` sampled rows
    (0: none), then the time-based warm-up and `steps` timed calls. Returns a
    small summary (TFLOP/s from the mean launch duration, fraction of the
    dense peak, the gate's error)."""
    import numpy as np
    from online_softmax_amd.inputs import make_qkv, sample_rows
    dev = torch.device("cuda:0")
    scale = 0.125
    q, k, v = make_qkv(B, H, T, 64, dtype, seed)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    run = lambda: osa.attn_fwd_stream(qd, kd, vd, o, lse, True, scale, stream)
    run()
    torch.cuda.synchronize()
    out = {"B": B, "H": H, "T": T}
    if gate_rows and oracle is not None:
        rows = sample_rows(B, H, T, gate_rows, seed + 77,
                           boundaries=(64, 128, T // 2))
        ro, rl = oracle.attention(q, k, v, True, scale, rows=rows,
                                  threads=oracle.max_threads())
        eo = float(np.abs(o.float().cpu().numpy().reshape(-1, 64)[rows] - ro).max())
        el = float(np.abs(lse.cpu().numpy().reshape(-1)[rows] - rl).max())
        ok = eo <= BF16_TOL and el <= BF16_TOL and bool(torch.isfinite(o.float()).all())
        out["gate"] = {"rows": int(len(rows)), "err_o": eo, "err_lse": el, "pass": ok}
        if not ok:
            log(f"forward {label or T}: correctness gate FAILED ({eo:.3e}, {el:.3e})")
            return out
    r = timed_calls(torch, run, stream, steps, warmup)
    flops = osa.attn_flops(B, H, T, 64, True)
    tf = flops / (r["mean"] * 1e-3) / 1e12
    out.update({"ms": r["mean"], "per_call_mean_ms": r["per_call_mean"],
                "median_ms": r["median"], "tflops": tf, "frac": tf / PEAK_TFLOPS[dtype],
                "device_pauses": r["device_pauses"]})
    log(f"forward {label or ''} B={B} H={H} T={T}: {r['mean']:.4f} ms per call back to back "
        f"(per-call events: mean {r['per_call_mean']:.4f}, median {r['median']:.4f}), "
        f"{tf:.1f} TFLOP/s = {100 * tf / PEAK_TFLOPS[dtype]:.1f}%"
        + (f", gate err {out['gate']['err_o']:.2e}" if "gate" in out else ""))
    del qd, kd, vd, o, lse
    return out


def context_leg(osa, torch, w, qd, kd, vd, steps=20):
    """Other programs on the same chip, for context (none is part of the
    path): torch's own fused attention (scaled_dot_product_attention,
    flash backend only, on the metric's inputs: the comparison the page
    "Flash attention in PyTorch, then in Triton" draws in section "A kernel
    in Triton"), and the vendor library's dense bf16 matrix product
    (torch.matmul, 8192^3, seeded N(0,1) operands), the matrix-core rate a
    plain GEMM reaches here, and a device copy of the decode leg's 100 MB
    (the rate plain streaming of those bytes reaches here). Only the flash
    backend is allowed: if it cannot run the call, the leg records why
    instead of falling back to the math path."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from online_softmax_amd.inputs import make_qkv
    stream = torch.cuda.current_stream()
    out = {}
    flops = osa.attn_flops(w.B, w.H, w.T, w.D, w.causal)
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            run = lambda: torch.nn.functional.scaled_dot_product_attention(
                qd, kd, vd, is_causal=w.causal, scale=w.scale)
            ref = run()
            r = timed_calls(torch, run, stream, steps)
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=qd.device)
        osa.attn_fwd_stream(qd, kd, vd, o, lse, w.causal, w.scale, stream)
        torch.cuda.synchronize()
        out["torch_sdpa"] = {"ms": r["mean"], "tflops": flops / (r["mean"] * 1e-3) / 1e12,
                             "max_abs_diff_to_ours": float((ref.float() - o.float()).abs().max())}
        del ref, o, lse
    except RuntimeError as e:
        out["torch_sdpa"] = {"error": str(e)[:200]}
    # forward + backward, the pair the page times for training (its flop
    # count: the forward's two products and the backward's five, 3.5 times
    # the forward's): ours through the entry points, torch's through its
    # flash backend and autograd
    (dout,) = make_qkv(w.B, w.H, w.T, w.D, w.dtype, 4243)[:1]
    dd = dout.to(qd.device)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=qd.device)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(osa.attn_bwd_workspace_bytes(w.B, w.H, w.T), dtype=torch.uint8,
                     device=qd.device)

    def ours_pair():
        osa.attn_fwd_stream(qd, kd, vd, o, lse, w.causal, w.scale, stream)
        osa.attn_bwd_stream(qd, kd, vd, o, dd, lse, dq, dk, dv, ws, w.causal, w.scale, stream)
    r = timed_calls(torch, ours_pair, stream, steps)
    pair_flops = 3.5 * flops
    out["fwd_bwd_ours"] = {"ms": r["mean"], "tflops": pair_flops / (r["mean"] * 1e-3) / 1e12}
    del o, lse, dq, dk, dv, ws
    try:
        qg, kg, vg = (x.detach().clone().requires_grad_() for x in (qd, kd, vd))

        def torch_pair():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                oo = torch.nn.functional.scaled_dot_product_attention(
                    qg, kg, vg, is_causal=w.causal, scale=w.scale)
            torch.autograd.grad(oo, (qg, kg, vg), dd)
        r = timed_calls(torch, torch_pair, stream, steps)
        out["fwd_bwd_torch_sdpa"] = {"ms": r["mean"],
                                     "tflops": pair_flops / (r["mean"] * 1e-3) / 1e12}
        del qg, kg, vg
    except RuntimeError as e:
        out["fwd_bwd_torch_sdpa"] = {"error": str(e)[:200]}
    del dd
    n = 8192
    g = torch.Generator(device="cpu").manual_seed(4242)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to(qd.device)
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to(qd.device)
    r = timed_calls(torch, lambda: torch.matmul(a, b), stream, steps)
    out["gemm_bf16_8192"] = {"ms": r["mean"], "tflops": 2 * n**3 / (r["mean"] * 1e-3) / 1e12}
    del a, b
    # what streaming reaches here at the decode leg's size: a device copy
    # (torch copy_) of 100,663,296 B (the K and V of the 4 x 12 x 8192 x 64
    # bf16 cache), rotating over four source/destination pairs (800 MB, past
    # the 256 MB Infinity Cache); bytes read plus bytes written per time
    nbytes = 2 * 4 * 12 * 8192 * 64 * 2
    srcs = [torch.ones(nbytes, dtype=torch.uint8, device=qd.device) for _ in range(4)]
    dsts = [torch.empty_like(x) for x in srcs]
    turn = [0]

    def copy():
        i = turn[0] % 4
        turn[0] += 1
        dsts[i].copy_(srcs[i])
    r = timed_calls(torch, copy, stream, 4 * steps)
    out["hbm_copy_100MB"] = {"us": r["mean"] * 1e3,
                             "GBs_read_plus_write": 2 * nbytes / (r["mean"] * 1e-3) / 1e9}
    del srcs, dsts
    torch.cuda.synchronize()
    s = out["torch_sdpa"]
    fb, tb = out["fwd_bwd_ours"], out["fwd_bwd_torch_sdpa"]
    log(f"context: forward + backward: ours {fb['ms']:.3f} ms ({fb['tflops']:.1f} TFLOP/s by "
        "the page's 3.5x count), torch SDPA (flash) "
        + (f"{tb['ms']:.3f} ms ({tb['tflops']:.1f})" if "ms" in tb else tb["error"]))
    log("context: torch SDPA (flash) " + (f"{s['ms']:.4f} ms, {s['tflops']:.1f} TFLOP/s"
                                           if "ms" in s else s["error"])
        + f"; bf16 GEMM 8192^3 {out['gemm_bf16_8192']['tflops']:.1f} TFLOP/s"
        + f"; device copy of 100 MB {out['hbm_copy_100MB']['us']:.1f} us "
          f"({out['hbm_copy_100MB']['GBs_read_plus_write']:.0f} GB/s read + write)")
    return out


def memory_contrast(osa, torch, w):
    """Device memory held by each forward path at the metric's B, H and T,
    measured by the caching allocator's peak around one call (the library
    allocates nothing itself; hipMemGetInfo around the call checks that):
    the fused path on the bf16 inputs, the naive path in fp32 (its T x T
    tables live in a caller-owned workspace)."""
    dev = torch.device("cuda:0")
    out = {}
    for path in ("fused", "naive"):
        dt = torch.bfloat16 if path == "fused" else torch.float32
        shape = (w.B, w.H, w.T, w.D)
        q, k, v = (torch.randn(shape, device=dev, dtype=torch.float32).to(dt) for _ in range(3))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        free0 = torch.cuda.mem_get_info(dev)[0]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
        if path == "fused":
            osa.attn_fwd_stream(q, k, v, o, lse, True, w.scale)
        else:
            ws = torch.empty(osa.attn_naive_workspace_bytes(w.B, w.H, w.T),
                             dtype=torch.uint8, device=dev)
            osa.attn_naive_fwd(q, k, v, o, lse, ws, True, w.scale)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev)
        free1 = torch.cuda.mem_get_info(dev)[0]
        out[path] = {"dtype": "bf16" if path == "fused" else "f32",
                     "inputs_B": base, "held_beyond_inputs_B": peak - base,
                     "output_B": o.numel() * o.element_size() + lse.numel() * 4,
                     "driver_free_drop_B": max(0, free0 - free1)}
        log(f"memory, {path} path at B={w.B} H={w.H} T={w.T}: inputs {base / 2**20:.1f} MiB, "
            f"held beyond them {(peak - base) / 2**20:.1f} MiB")
        del q, k, v, o, lse
        if path == "naive":
            del ws
    # forward + backward through flash_attention (the training pair the page
    # measures memory for): what autograd and the library hold beyond the
    # inputs and the output gradient (O, lse, dQ, dK, dV, the backward's
    # workspace of two floats per row)
    shape = (w.B, w.H, w.T, w.D)
    q, k, v = (torch.randn(shape, device=dev, dtype=torch.float32).to(torch.bfloat16)
               .requires_grad_() for _ in range(3))
    dout = torch.randn(shape, device=dev, dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    grads = torch.autograd.grad(osa.flash_attention(q, k, v, True, w.scale), (q, k, v), dout)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    out["fused_fwd_bwd"] = {"dtype": "bf16", "inputs_B": base,
                            "held_beyond_inputs_B": peak - base}
    log(f"memory, fused forward + backward at B={w.B} H={w.H} T={w.T}: held beyond the "
        f"inputs and dO {(peak - base) / 2**20:.1f} MiB")
    del q, k, v, dout, grads
    torch.cuda.empty_cache()
    return out


def compact(d, nd=4):
    """Round floats for the one-line summary."""
    if isinstance(d, float):
        return float(f"{d:.{nd}g}")
    if isinstance(d, dict):
        return {k: compact(v, nd) for k, v in d.items()}
    if isinstance(d, (list, tuple)):
        return [compact(v, nd) for v in d]
    return d


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="warm-up calls (at least; warm-up also lasts at least "
                         "300 ms of device time)")
    ap.add_argument("--workload", default=None,
                    help="a name from online_softmax_amd.inputs.WORKLOADS")
    ap.add_argument("--cpu-rows", type=int, default=196608,
                    help="oracle sample size for the CPU baseline")
    ap.add_argument("--detail", default=None,
                    help="also write every figure of the run to this JSON file")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contrast", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sequence-length sweep and the long context")
    ap.add_argument("--no-131k", action="store_true",
                    help="skip the 131072-token long-context case (1 x 16 heads)")
    ap.add_argument("--no-memory", action="store_true",
                    help="skip the fused/naive device-memory contrast")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass leg")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode (key/value cache) leg")
    ap.add_argument("--no-head-dims", action="store_true",
                    help="skip the head dimension 32 / 128 legs")
    ap.add_argument("--no-recurrence", action="store_true",
                    help="skip the gated linear recurrence leg")
    ap.add_argument("--no-context", action="store_true",
                    help="skip timing torch's own fused attention and a bf16 GEMM")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB "
                         "(reference kernel for PMC byte counters)")
    a = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE {world}): the attention forward of one GPU's share "
              "is the whole workload here; no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_amd as osa
    from online_softmax_amd.inputs import METRIC_WORKLOAD, WORKLOADS, workload_qkv
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    osa.load()
    w = WORKLOADS[a.workload or METRIC_WORKLOAD]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"GPU: {props.name} ({props.gcnArchName}), {props.multi_processor_count} CUs")
    traffic_f, _ = print_traffic(osa, w)
    kernels = print_kernel_table(osa)

    q, k, v = workload_qkv(w)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    osa.attn_fwd_stream(qd, kd, vd, o, lse, w.causal, w.scale)
    torch.cuda.synchronize()

    oracle = None
    if not a.no_cpu_baseline:
        import oracle
    cpu, parity = None, None
    if oracle is not None:
        log(f"oracle on {a.cpu_rows} sampled rows (correctness gate and CPU "
            "baseline) ...")
        cpu, parity = cpu_baseline(oracle, q, k, v, o, lse, w, a.cpu_rows, 9001)
        bound = BF16_TOL if w.dtype != "f32" else max(
            F32_TOL_BASE, F32_TOL_BASE * math.sqrt(w.T / 256))
        parity["bound"] = bound
        parity["pass"] = (parity["finite"] and parity["max_abs_err_o"] <= bound
                          and parity["max_abs_err_lse"] <= bound)
        log(f"  parity on sample: {parity}")
        log(f"  oracle: {cpu['value'] * 1e3:.2f} GFLOP/s ({cpu['sample']})")
        if not parity["pass"]:
            log("correctness gate FAILED: not timing a wrong kernel")
            sys.exit(3)

    # The headline: W warm-up calls (and at least 300 ms of them), then K
    # timed steps bracketed by synchronisation.
    stream = torch.cuda.current_stream()
    run = lambda: osa.attn_fwd_stream(qd, kd, vd, o, lse, w.causal, w.scale, stream)
    warm_calls, warm_ms = warm_up(torch, run, stream, a.warmup)
    t = time_steps(torch, run, stream, a.steps)
    flops = osa.attn_flops(w.B, w.H, w.T, w.D, w.causal)
    value = flops / (t["wall_ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (t["mean"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"fused: warm-up {warm_calls} calls ({warm_ms:.0f} ms); {t['wall_ms_per_step']:.4f} "
        f"ms/step wall, launch mean {t['mean']:.4f} ms (median {t['median']:.4f}, min "
        f"{t['min']:.4f}, max {t['max']:.4f}); {t['device_pauses']} device pauses, "
        f"{t['host_ms']:.3f} ms host-side; {achieved:.1f} TFLOP/s = "
        f"{100 * achieved / peak:.1f}% of {peak} TFLOP/s")
    del o, lse

    ctx = None
    if not a.no_context and w.dtype != "f32":
        ctx = context_leg(osa, torch, w, qd, kd, vd)

    sweep = long_ctx = None
    if not a.no_sweep and w.name == METRIC_WORKLOAD:
        sweep = {}
        for T in (1024, 2048, 4096, 8192, 16384):
            sweep[str(T)] = forward_case(osa, torch, oracle, 4, 12, T, "bf16", 2500 + T,
                                         steps=100 if T <= 2048 else 20, warmup=20,
                                         label="sweep")
        long_ctx = {}
        for name in ("long_b1h16_t32768_bf16",) + (("long_b1h16_t131072_bf16",)
                                                   if not a.no_131k else ()):
            lw = WORKLOADS[name]
            long_ctx[str(lw.T)] = forward_case(
                osa, torch, oracle, lw.B, lw.H, lw.T, lw.dtype, lw.seed,
                steps=10 if lw.T <= 32768 else 3, warmup=3, gate_rows=4096, label=name)

    mem = None
    if not a.no_memory:
        mem = memory_contrast(osa, torch, w)

    if a.copy_mib > 0:  # reference kernel of known size for byte counters
        src = torch.empty(a.copy_mib * 2**20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {a.copy_mib} MiB x 3 (PMC reference)")
        del src, dst

    bwd = bwd_atomic = None
    if not a.no_backward and w.dtype != "f32":
        cache = {}
        bwd = backward_leg(osa, torch, oracle, w, q, k, v, qd, kd, vd, *fresh_out(osa, torch, qd, kd, vd, w),
                           with_oracle=oracle is not None, cache=cache)
        bwd_atomic = backward_leg(osa, torch, oracle, w, q, k, v, qd, kd, vd,
                                  *fresh_out(osa, torch, qd, kd, vd, w),
                                  with_oracle=oracle is not None, atomic=True, cache=cache)
        bwd_atomic.pop("cpu_baseline", None)

    dec = dec128 = None
    if not a.no_decode:
        dec = decode_leg(osa, torch, oracle, with_oracle=oracle is not None)
        dec128 = decode_leg(osa, torch, oracle, D=128, with_oracle=oracle is not None)
        dec128.pop("cpu_baseline", None)

    hds = None
    if not a.no_head_dims:
        hds = {str(D): head_dim_leg(osa, torch, oracle, D, with_oracle=oracle is not None)
               for D in (32, 128)}

    recur = None
    if not a.no_recurrence:
        recur = recurrence_leg(osa, torch, oracle, with_oracle=oracle is not None)

    extra = None
    if not a.no_contrast and oracle is not None:
        extra = contrast(osa, torch, oracle)

    single = None
    if oracle is not None:
        single = oracle_single_core(oracle)

    dt_code = {"f32": osa.ATTN_F32, "bf16": osa.ATTN_BF16, "f16": osa.ATTN_F16}[w.dtype]
    kname = osa.attn_kernel_name(osa.attn_fused_kernel(w.B, w.H, w.T, w.D, w.causal, dt_code))
    roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": measured_traffic(), "kernel": kname,
                "launch_ms": {"mean": t["mean"], "median": t["median"]}}
    detail = {
        "metric": METRIC, "value": value, "warmup_calls": warm_calls, "warmup_ms": warm_ms,
        "timing": t, "roofline": dict(roofline, algorithmic_flop_per_launch=flops,
                                      traffic_arith_B=traffic_f),
        "cpu_baseline": cpu, "parity": parity, "kernels": kernels, "sweep": sweep,
        "long_context": long_ctx, "memory": mem, "backward": bwd,
        "backward_atomic": bwd_atomic, "cpu_single_core": single, "decode": dec,
        "decode_d128": dec128, "head_dims": hds, "gated_recurrence": recur,
        "contrast_fp32_single_head": extra, "context": ctx,
        "kernel_source_sha256": kernel_source_hash()}
    log("bench detail: " + json.dumps(detail))
    if a.detail:
        with open(a.detail, "w") as f:
            json.dump(detail, f, indent=1)

    def leg(x, key="roofline"):
        if not x or not x.get("pass", True) or key not in x:
            return None if not x else {"pass": x.get("pass")}
        r = x[key]
        return [r["achieved"], r["unit"], r["frac"]]

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "warmup_calls": warm_calls,
        "ms_per_step": t["wall_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": f"synthetic: seeded N(0,1) fp32 rounded to {w.dtype}",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
                   "causal": w.causal, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {
            "value": cpu["value"], "unit": cpu["unit"], "cores": cpu["cores"],
            "kind": "oracle", "sample": f"{parity['rows']} seeded rows of {w.name}"},
        "parity": None if parity is None else
            f"{parity['rows']} rows vs oracle: max|dO| {parity['max_abs_err_o']:.2e}, "
            f"max|dlse| {parity['max_abs_err_lse']:.2e}, bound {parity['bound']:g}, "
            + ("pass" if parity["pass"] else "FAIL"),
        "pauses": {"device": t["device_pauses"], "host_ms": t["host_ms"]},
        "sweep_tflops": None if sweep is None else
            {T: s.get("tflops") for T, s in sweep.items()},
        "long_context": None if long_ctx is None else
            {T: {"tflops": s.get("tflops"), "frac": s.get("frac"),
                 "gate_err": s.get("gate", {}).get("err_o")} for T, s in long_ctx.items()},
        "memory_beyond_inputs_B": None if mem is None else
            {p: m["held_beyond_inputs_B"] for p, m in mem.items()},
        "legs": {"bwd": leg(bwd), "bwd_atomic": leg(bwd_atomic), "decode": leg(dec),
                 "decode_noalloc": leg((dec or {}).get("noalloc")),
                 "decode_graph": None if not dec or "graph_replay_GBs" not in dec else
                     [dec["graph_replay_GBs"], "GB/s", dec["graph_replay_GBs"] / PEAK_HBM_GBS],
                 "decode_d128": leg(dec128),
                 "d32": leg((hds or {}).get("32")), "d128": leg((hds or {}).get("128")),
                 "recurrence": leg((recur or {}).get("throughput"))},
        "context_tflops": None if ctx is None else
            {"torch_sdpa_flash": ctx["torch_sdpa"].get("tflops"),
             "fwd_bwd_ours": ctx["fwd_bwd_ours"]["tflops"],
             "fwd_bwd_torch_sdpa_flash": ctx["fwd_bwd_torch_sdpa"].get("tflops"),
             "gemm_bf16_8192": ctx["gemm_bf16_8192"]["tflops"],
             "hbm_copy_100MB_GBs": ctx["hbm_copy_100MB"]["GBs_read_plus_write"]},
    }
    sys.stderr.flush()
    print(json.dumps(compact(line), separators=(",", ":")), flush=True)


def fresh_out(osa, torch, qd, kd, vd, w):
    """O and lse of the metric workload for the backward legs."""
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=qd.device)
    osa.attn_fwd_stream(qd, kd, vd, o, lse, w.causal, w.scale)
    torch.cuda.synchronize()
    return o, lse


if __name__ == "__main__":
    main()
