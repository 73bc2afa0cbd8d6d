"""bench.py's contract pieces that need no GPU: one GPU only (--gpus above 1 exits with a message
before touching the GPU), and the HBM-traffic figure is used only when the committed counter
measurement was taken on the current kernel sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() == 123.0
    rec["kernel_source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_kernel_source_hash_covers_the_gemm_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    # the hash follows the GEMM kernel's source text
    csrc = tmp_path / "block_scaled_fp8_grouped_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("gemm.hip", "common.hpp", "group_layout.hpp", "tile_addr.hpp", "tile_sched.hpp"):
        src = os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "csrc", name)
        (csrc / name).write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash() == h
    (csrc / "gemm.hip").write_bytes((csrc / "gemm.hip").read_bytes() + b"\n")
    assert bench.kernel_source_hash() != h
