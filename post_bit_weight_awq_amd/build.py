"""Builds libawq_mi355x.so (gfx950 only) in the package directory with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq_mi355x.so")
SOURCES = ["act_stats.hip", "search.hip", "search_grid.hip", "search_gemm.hip", "pack.hip",
           "w4a16.hip", "fold.hip", "select.hip", "awq_api.hip"]
# measured-peak references used by bench.py only (not part of the search library)
CALIB_LIB = os.path.join(PKG, "libawq_calib.so")
CALIB_SOURCES = ["calib.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # no packed fp32 VALU ops anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE binary32 division and denormals: the codes depend on them
    "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "-save-temps")
        objs.append(obj)
        cmds.append(cmd)
    cwd = os.getcwd()
    if save_temps:
        os.chdir(BUILD)
    try:
        with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
            outs = list(ex.map(_run, cmds))
    finally:
        os.chdir(cwd)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    ctmp = CALIB_LIB + ".tmp"
    _run([cc, *HIPCC_FLAGS, "-shared", "-o", ctmp,
          *[os.path.join(CSRC, s) for s in CALIB_SOURCES]])
    os.replace(ctmp, CALIB_LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
