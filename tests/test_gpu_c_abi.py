"""The C ABI from plain C, with no Python or torch in the process: tests/host/c_abi_gpu.c allocates
device memory with the HIP runtime, sizes it with the library's size queries, quantizes dy and x
(MXFP8 colwise) and runs the k-grouped weight gradient through include/bsfp8.h, and checks the
bytes against the oracle bit for bit and each expert's gradient within 1e-5 relative Frobenius
error (groups of 200, 0, 33 and 128 rows, garbage padding rows)."""
import subprocess

import pytest

from c_abi_build import exe
from gpu_util import flush

pytestmark = pytest.mark.gpu


def test_plain_c_caller():
    flush("plain C caller of libbsfp8.so")
    r = subprocess.run([exe()], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("PASS"), r.stdout
