"""Compile libstarkv.so (HIP, gfx950) in-tree with hipcc.

    python -m rank_compressed_paged_amd.build

Each source is compiled to an object file in its own hipcc process (in
parallel), then the objects are linked into the shared library.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstarkv.so")
SOURCES = ["starkv_api.hip", "decode_kernels.hip", "attn_dispatch.hip", "attn_inst_exact.hip", "attn_inst_mha.hip",
           "attn_inst_gqa.hip", "append_kernels.hip", "prefill_kernels.hip", "uncompressed_kernels.hip",
           "probe_kernels.hip"]
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # packed fp32 VALU ops stay off on this target (float code is emitted unpacked)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def compile_command(src: str, obj: str) -> list:
    return [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, errs


def build(verbose: bool = False, jobs: int | None = None) -> str:
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="starkv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_command(s, o) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for src, (rc, errs) in zip(SOURCES, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{errs}")
            if verbose and errs.strip():
                print(errs, file=sys.stderr)
        tmp_lib = LIB + ".tmp"
        cmd = link_command(objs, tmp_lib)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, errs = _run(cmd)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
