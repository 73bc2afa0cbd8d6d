"""Host sweep of the per-group colwise layout header (csrc/group_layout.hpp) that the quantize
kernels write through and the GEMM kernels and size queries read through: writer and reader
offsets agree, every element, E8M0 byte and fp32 scale has exactly one place, pad lanes
included, over ragged, empty and 1024-group splits (TE PR #3224, Greptile summary: per-member
columnwise scale strides)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_group_layout_sweep(tmp_path):
    exe = tmp_path / "group_layout_check"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I",
                           os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "csrc"),
                           os.path.join(ROOT, "tests", "host", "group_layout_check.cpp"), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
