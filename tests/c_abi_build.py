"""Build of the plain-C GPU caller tests/host/c_abi_gpu.c (test infrastructure: it links the
oracle) into _build/c_abi_gpu, with gcc against the HIP runtime, libbsfp8.so and liboracle.so."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "c_abi_gpu.c")
EXE = os.path.join(ROOT, "_build", "c_abi_gpu")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "block_scaled_fp8_grouped_amd"), "-lbsfp8",
           "-L", os.path.join(ROOT, "oracle"), "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-fopenmp", "-Wl,-rpath,$ORIGIN/../block_scaled_fp8_grouped_amd", "-Wl,-rpath,$ORIGIN/../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


def exe():
    """The built caller, rebuilt when missing or older than its source or the header."""
    hdr = os.path.join(ROOT, "include", "bsfp8.h")
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(SRC), os.path.getmtime(hdr)):
        build()
    return EXE
