"""CPU check of every index the fused kernels form (bounds, alignment, LDS
coverage, tile bijection, P/V key pairing), by compiling tests/layout_check.cpp
against the kernels' own index header with the host compiler."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fused_kernel_indices(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "online_softmax_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "layout ok" in r.stdout
