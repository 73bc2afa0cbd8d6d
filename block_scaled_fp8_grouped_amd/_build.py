"""Build of libbsfp8.so (gfx950) with hipcc, in-tree.

Every HIP source is compiled with IEEE fp32 semantics for the quantize arithmetic (no FMA
contraction, correctly rounded fp32 division) and without packed-fp32 instruction selection.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libbsfp8.so")
SOURCES = ["bsfp8.cpp", "quantize.hip", "gemm.hip"]
# the MFMA-only throughput probe, a library of its own (measurement, not the path)
PEAK_LIB_PATH = os.path.join(HERE, "libbsfp8_peak.so")
PEAK_SOURCES = ["mfma_peak.hip"]
HEADERS = ["common.hpp", "group_layout.hpp", "tile_addr.hpp", "tile_sched.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, obj):
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, path)


def build(verbose=True):
    """Compile every source for gfx950 and link libbsfp8.so (and the probe libbsfp8_peak.so)
    next to this file."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        list(ex.map(_compile, srcs, objs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PEAK_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PEAK_LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
