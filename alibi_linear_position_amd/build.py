"""Build libalibi.so in-tree with hipcc for gfx950.

    python -m alibi_linear_position_amd.build          # or build() from Python

Every HIP source under csrc/ is compiled with -O3 for gfx950 only, with the
packed-fp32 instruction feature disabled, and linked into one shared library
next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libalibi.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "fwd_generic.hip", "fwd_mfma.hip", "decode.hip", "knorm.hip", "bwd.hip",
           "stream_read.hip", "mfma_rate.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libalibi)")


def compile_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-I", INCLUDE, "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False, out: str = LIB, extra_flags=(), jobs: int = 0) -> str:
    """Compile every source and link the shared library (libalibi.so next to
    this file by default); returns its path. extra_flags are added to every
    compile and to the link (e.g. host-only instrumentation of a test build);
    jobs: parallel compiles (0 = one per available core, at most 8)."""
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    extra = list(extra_flags)
    if jobs <= 0:
        jobs = max(1, min(8, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="alibi_build_") as tmp:
        cmds = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmds.append([cc, *compile_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(max_workers=jobs) as pool:
            list(pool.map(run, cmds))
        tmp_lib = out + ".tmp"
        run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp_lib])
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
