"""bench.py end to end on the GPU, cut to one step and a tiny CPU sample: it prints exactly one JSON
line on stdout with the fields and types its contract names (the headline metric, the roofline
object of the wgrad kernel, the CPU-oracle baseline), and the figures are consistent."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import flush

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    flush("bench.py one step")
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "1", "--no-graph",
           "--no-mxfp4", "--cpu-experts", "1", "--cpu-channels", "64", "--no-config-oracle"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[k], t), (k, d.get(k))
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 1 and d["unit"] == "TFLOP/s"
    assert d["vs_baseline"] is None and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 5000.0  # the FP8 MFMA peak
    assert abs(rf["frac_of_bf16_peak"] - rf["achieved"] / 2500.0) < 1e-3
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    # value counts the whole step, so it cannot exceed the wgrad kernel's own rate
    assert 0 < d["value"] <= rf["achieved"]
    # the other four workloads, timed on the GPU
    cf = d["configs"]
    assert sorted(cf) == ["1_deepgemm_256_padded", "2_te3484_single_group", "3_deepgemm_2048", "4_moe32_zipf"]
    for name, legs in cf.items():
        assert legs["wgrad"]["us"] > 0 and legs["wgrad"]["GB/s"] > 0, name
    assert cf["4_moe32_zipf"]["fprop"]["TFLOP/s"] > 0
    # the fp8-MFMA leg: its rate and its measured error next to the widened path's
    f8 = d["fp8_mfma"]
    assert f8["wgrad_TFLOP/s"] > 0 and abs(f8["wgrad_frac_of_fp8_peak"] - f8["wgrad_TFLOP/s"] / 5000.0) < 1e-3
    assert f8["rel_err_vs_oracle"]["bf16_widened"] <= 1e-5 < f8["rel_err_vs_oracle"]["fp8_mfma"] <= 5e-5
    # the vendor library's dense GEMMs on one expert's shape, beside the grouped kernel
    lib = d["library_reference"]
    assert lib["bf16_TFLOP/s"] > 0 and abs(lib["wgrad_vs_bf16"] - rf["achieved"] / lib["bf16_TFLOP/s"]) < 2e-3
    assert "fp8_TFLOP/s" in lib or "fp8_error" in lib
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["cores"] >= 1 and cb["value"] > 0
    assert isinstance(cb["sample"], str) and cb["sample"]
