"""The forward's workgroup map, checked on the CPU (no GPU).

The kernels find their work from the workgroup id: map_item in
csrc/kernel_common.h picks the (batch, KV head, head group) unit, the row
block (two mirror blocks when the row blocks are folded) and the key range;
item_row and slot_head place each of the 128 query slots. This builds
tests/workmap_check.cpp with hipcc as a host program, which maps every
workgroup of the grid for 25 shapes (MHA, GQA, MQA, decode, ragged and
single-row cases) with and without a causal mask, unsplit and with three key
ranges, folded and unfolded, and checks that every (batch, query head, row,
key range) is held by exactly one slot.
"""

import os
import subprocess
import tempfile

import pytest

from tests.test_fastdiv import CSRC, HERE, _hipcc


def test_workgroup_map_covers_every_row_once():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "workmap_check")
        subprocess.run([hipcc, "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "workmap_check.cpp"), "-o", exe],
                       check=True, capture_output=True, text=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        print(r.stdout)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "failures 0" in r.stdout
