"""Build libfox.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m forget_gated_causal_amd.build`` (or ``build()`` from Python).
Every call recompiles; objects go to ``_build/`` at the repository root and the
shared library to ``forget_gated_causal_amd/libfox.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfox.so")
SOURCES = ["fox_api.hip", "fox_scan.hip", "fox_fwd.hip", "fox_decode.hip", "fox_bwd.hip", "fox_bwd_f32.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    extra = ["-save-temps=obj"] if save_temps else []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([cc, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
