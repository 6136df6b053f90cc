"""Build libattn.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m online_softmax_amd.build           # compile
    python -m online_softmax_amd.build --asm     # also write gfx950 assembly

The library is compiled every time build() is called. Packed fp32 vector
instructions are disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "fused_fwd.hip", "naive_fwd.hip", "attn_bwd.hip",
           "attn_bwd_atomic.hip", "attn_decode.hip", "fused_hd.hip",
           "recurrence.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel) and link libattn.so;
    returns its path."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="attn_build_") as objdir:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            cmd = [hipcc(), *flags(), "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((src, subprocess.Popen(cmd)))
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(failed))
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-fPIC", "-shared", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def assembly(source: str, out: str) -> str:
    """Device assembly of one source for gfx950 (for inspection)."""
    cmd = [hipcc(), *flags(), "--cuda-device-only", "-S", "-o", out,
           os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", metavar="DIR", default=None,
                    help="also write device assembly of each source to DIR")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.verbose))
    if a.asm:
        os.makedirs(a.asm, exist_ok=True)
        for s in SOURCES:
            print(assembly(s, os.path.join(a.asm, s.replace(".hip", ".s"))))
