"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

No GPU is needed.  A copy of the library is built whose host code (argument
checks, workspace layouts, launch set-up) carries both sanitizers; the device
code is built as usual.  The host ABI tests then run against that copy in a
child Python with the shared ASan runtime preloaded.  Any sanitizer report
ends the child with an error and fails this test.
"""

import os
import subprocess
import sys

import pytest

from rank_compressed_paged_amd import build as starkv_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    lib = starkv_build.build(out=str(tmp_path / "libstarkv_host_sanitized.so"), host_sanitize=True)
    env = dict(os.environ)
    preload = [starkv_build.host_asan_runtime()]
    if env.get("LD_PRELOAD"):
        preload.append(env["LD_PRELOAD"])      # the ASan runtime must come first
    env.update({
        "STARKV_LIBRARY": lib,
        "LD_PRELOAD": ":".join(preload),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q", "-s",
           "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    reports = [l for l in out.splitlines() if "runtime error" in l or "ERROR: AddressSanitizer" in l]
    assert r.returncode == 0 and not reports, "\n".join(reports[:5] or out.splitlines()[-40:])
    assert " passed" in out
