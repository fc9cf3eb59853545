"""Compile libstarkv.so (HIP, gfx950) in-tree with hipcc.

    python -m rank_compressed_paged_amd.build
    python -m rank_compressed_paged_amd.build --host-sanitize OUT.so

Each source is compiled to an object file in its own hipcc process (in
parallel), then the objects are linked into the shared library.  The second
form builds a copy whose host code (argument checks, layouts, launch set-up)
carries AddressSanitizer and UndefinedBehaviorSanitizer; the device code is
built as usual.  Load it with the ASan runtime preloaded (host_asan_runtime()).
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


# host-side sanitizers only (each -fsanitize= applies to the host pass alone)
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
HOST_SANITIZE_COMPILE = HOST_SANITIZE + "-Xarch_host -fno-sanitize-recover=undefined -g".split()


def compile_command(src: str, obj: str, extra: tuple = ()) -> list:
    return [hipcc(), *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str, extra: tuple = ()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", out]


def host_asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to LD_PRELOAD into Python)."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        cands = sorted(glob.glob(os.path.join(rocm, "llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")))
        if not cands:
            raise RuntimeError("no shared ASan runtime found next to hipcc")
        out = cands[-1]
    return out


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, errs


def build(verbose: bool = False, jobs: int | None = None, out: str = LIB, host_sanitize: bool = False) -> str:
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    cflags = tuple(HOST_SANITIZE_COMPILE) if host_sanitize else ()
    lflags = tuple(["-shared-libasan", *HOST_SANITIZE]) if host_sanitize else ()
    with tempfile.TemporaryDirectory(prefix="starkv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_command(s, o, cflags) for s, o in zip(SOURCES, objs)]
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
        tmp_lib = out + ".tmp"
        cmd = link_command(objs, tmp_lib, lflags)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, errs = _run(cmd)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-sanitize":
        print(build(verbose=True, out=os.path.abspath(sys.argv[2]), host_sanitize=True))
    else:
        print(build(verbose=True))
