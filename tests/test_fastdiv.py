"""The workgroup map's division by launch-time multipliers (CPU only).

The kernels divide workgroup and slot indices by launch constants with the
round-up multiplier method (FastDiv in csrc/kernel_common.h): the host
computes the multiplier, the device a multiply, an add and a shift. This
builds tests/fastdiv_check.cpp with hipcc as a host program and checks the
quotient against integer division over every dividend below 8192 for every
divisor up to 4096, the ends of the dividend range, multiples of the divisor
and their neighbours, and random divisor / dividend pairs below 2^31.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "scaled_dot_product_09_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_fastdiv_matches_integer_division():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "fastdiv_check")
        subprocess.run([hipcc, "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "fastdiv_check.cpp"), "-o", exe],
                       check=True, capture_output=True, text=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        print(r.stdout)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "mismatches 0" in r.stdout
