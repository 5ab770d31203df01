"""Build of the HIP library ``libmixq.so`` for gfx950 (hipcc, in-tree).

Each source is compiled to an object in parallel, then the objects are
linked into one shared library."""
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
LIB = os.path.join(PKG, "libmixq.so")
SOURCES = ["mixq_api.hip", "mixq_act.hip", "mixq_weight.hip", "mixq_gemm.hip", "mixq_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    with tempfile.TemporaryDirectory(prefix="mixq_build_") as tmpdir:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            subprocess.run(cmd, check=True)
            return obj

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
