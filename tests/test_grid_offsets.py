"""Host-side range check of the fused grid kernels' index arithmetic.

The kernels address every load as a uniform 64-bit base plus a per-lane
32-bit offset, and map each block to a (grid point, tile) unit.  Those
formulas live in post_bit_weight_awq_amd/csrc/grid_index.h, which the kernels
include; tests/grid_offsets_check.cpp evaluates the same functions on the host
for shapes up to the largest the library accepts and checks that no offset
wraps or leaves its buffer and that every unit is covered exactly once.  No
GPU is involved.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_bit_weight_awq_amd", "csrc")


def _cxx():
    for c in ("g++", "c++", "clang++"):
        p = shutil.which(c)
        if p:
            return p
    pytest.skip("no host C++ compiler")


def test_grid_offsets_in_range(tmp_path):
    exe = str(tmp_path / "grid_offsets_check")
    subprocess.run([_cxx(), "-std=c++17", "-O2", "-I", CSRC,
                    os.path.join(ROOT, "tests", "grid_offsets_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:]


def test_grid_kernels_use_the_checked_index_helpers():
    """The grid kernels take their unit mapping and load offsets from the
    checked header rather than from formulas of their own."""
    src = open(os.path.join(CSRC, "search_grid.hip")).read()
    assert '#include "grid_index.h"' in src
    for fn in ("unit_of_block", "pp_act_offset", "pp_w_offset", "pp_param_offset",
               "pp_scale_offset", "g_act_offset", "g_w_offset", "g_param_offset"):
        assert re.search(r"gidx::%s\(" % fn, src), fn
    # no second copy of the mapping in the kernels
    assert "jb % n_grid" not in src
    gemm = open(os.path.join(CSRC, "search_gemm.hip")).read()
    assert '#include "grid_index.h"' in gemm
    for fn in ("gemm_unit_of_block", "gemm_offset"):
        assert re.search(r"gidx::%s\(" % fn, gemm), fn
