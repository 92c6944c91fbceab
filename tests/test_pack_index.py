"""Host-side check of the pack kernel's work mapping.

The pack kernel takes its launch plan, its lanes' first pairs, piece indices,
scale columns and load clamp from post_bit_weight_awq_amd/csrc/pack_index.h;
tests/pack_index_check.cpp evaluates the same functions on the host for every
group size and shapes up to the largest the library accepts, and on shapes
small enough to enumerate runs the kernel's sweep loop, checking that every
(row, group) pair is packed exactly once and every load and store stays in
its buffer.  No GPU is involved.
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


def test_pack_mapping_covers_every_pair_once(tmp_path):
    exe = str(tmp_path / "pack_index_check")
    subprocess.run([_cxx(), "-std=c++17", "-O2", "-I", CSRC,
                    os.path.join(ROOT, "tests", "pack_index_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:]


def test_pack_kernel_uses_the_checked_index_helpers():
    src = open(os.path.join(CSRC, "pack.hip")).read()
    assert '#include "pack_index.h"' in src
    for fn in ("plan", "first_pair", "piece_index", "first_column", "last_piece_index"):
        assert re.search(r"pidx::%s\(" % fn, src), fn
