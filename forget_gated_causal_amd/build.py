"""Build libfox.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m forget_gated_causal_amd.build`` (or ``build()`` from Python).
Every call recompiles; objects go to ``_build/`` at the repository root and the
shared library to ``forget_gated_causal_amd/libfox.so``.

``python -m forget_gated_causal_amd.build --host-sanitizers`` also builds
``_build/libfox_hostsan.so``: the same kernels, with the host layer (fox_api.hip: argument
checks, workspace carving, launches) under AddressSanitizer and UndefinedBehaviorSanitizer.
It is a check build, loaded through FOX_LIBRARY with the ASan runtime preloaded
(``host_sanitizer_env()``); device code is never instrumented.
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
SOURCES = ["fox_api.hip", "fox_scan.hip", "fox_fwd.hip", "fox_fwd_f32.hip", "fox_decode.hip", "fox_bwd.hip",
           "fox_bwd_f32.hip"]
# Per-source flags.  For a kernel with more than 256 registers (one wave per SIMD) the compiler
# puts every MFMA in AGPR form, and the scores then reach the VALU through AGPR-to-VGPR copies.
# The VGPR form is forced instead: fox_bwd.hip keeps its d = 128 accumulators in AGPRs by inline
# assembly, and fox_fwd.hip's one-wave kernels (4-wave blocks at d = 128) then fit 256 VGPRs.  The
# fp32 forward (fox_fwd_f32.hip) keeps the default: at d = 128 it needs the AGPRs.
SOURCE_FLAGS = {"fox_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
                "fox_fwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Host-only sanitizers: every -fsanitize= goes to the host pass alone.
HOST_SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]
HOSTSAN_LIB = os.path.join(BUILD, "libfox_hostsan.so")


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
        out = _run([cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (which also carries the UBSan handlers)."""
    out = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's shared ASan runtime not found")
    return path


def build_host_sanitized() -> str:
    """libfox with fox_api.hip's host code instrumented; the kernel objects are build()'s."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        if src == "fox_api.hip":
            obj = os.path.join(BUILD, "fox_api_hostsan.o")
            _run([cc, *HIP_FLAGS, *HOST_SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            if not os.path.exists(obj):
                _run([cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = HOSTSAN_LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN_FLAGS, *objs, "-o", tmp])
    os.replace(tmp, HOSTSAN_LIB)
    return HOSTSAN_LIB


def host_sanitizer_env(env=None) -> dict:
    """Environment for a child process that loads the sanitized build instead of libfox.so."""
    e = dict(os.environ if env is None else env)
    e["FOX_LIBRARY"] = HOSTSAN_LIB
    e["LD_PRELOAD"] = asan_runtime()
    # Python itself is not built with ASan: leaks at exit and its allocator are not ours.
    e["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    e["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return e


if __name__ == "__main__":
    print(build(verbose=True))
    if "--host-sanitizers" in sys.argv[1:]:
        print(build_host_sanitized())
