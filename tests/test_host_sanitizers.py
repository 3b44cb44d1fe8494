"""The host layer of libfox (fox_api.hip: argument checks, alias checks, workspace sizing and
carving) under AddressSanitizer and UndefinedBehaviorSanitizer.

The check build (``build.build_host_sanitized``) instruments only the host pass of fox_api.hip;
the kernels are the ordinary objects and are never launched here.  The host ABI tests run in a
child process that loads that build through FOX_LIBRARY with clang's ASan runtime preloaded; any
sanitizer report aborts the child.
"""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from forget_gated_causal_amd import build as fb

    try:
        fb.hipcc()
        fb.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    fb.build_host_sanitized()
    env = fb.host_sanitizer_env()
    log = str(tmp_path / "san")
    env["ASAN_OPTIONS"] += f":log_path={log}"
    env["UBSAN_OPTIONS"] += f":log_path={log}"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path) if f.startswith("san"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], reports[:3000])
