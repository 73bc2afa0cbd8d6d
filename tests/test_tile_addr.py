"""Host checks of the GEMM kernels' index arithmetic (the headers the kernels include), on the CPU:
* operand loads: every DMA source range inside its operand, every tile row/chunk delivered once
  to the LDS slot the fragment reads use, the E8M0 scale rows in range;
* tile order: the XCD-aware launch order produces every tile exactly once."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_load_addresses_in_bounds(tmp_path):
    exe = tmp_path / "tile_addr_check"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I",
                           os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "csrc"),
                           os.path.join(ROOT, "tests", "host", "tile_addr_check.cpp"), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout


def test_tile_order_is_a_bijection(tmp_path):
    exe = tmp_path / "tile_sched_check"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I",
                           os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "csrc"),
                           os.path.join(ROOT, "tests", "host", "tile_sched_check.cpp"), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
