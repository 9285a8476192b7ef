"""Host check of the grouped-GEMM tile schedule: the header that the GPU
kernels include is compiled with the host compiler and every workgroup's
unit is enumerated (coverage, disjoint K ranges, grid bound, block order)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_schedule_covers_every_tile_once(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "sched_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-I",
                    os.path.join(ROOT, "mixture_experts_layer_bincount_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "sched_check.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
