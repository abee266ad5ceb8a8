"""Build libtcgemm.so in-tree with hipcc for gfx950.

    python -m dense_gemm_tiled_amd.build        # or __graft_entry__.build()

Each source compiles to an object in parallel, then one shared library is
linked next to this file.  All HIP code is built with packed-fp32 instruction
selection switched off.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
from typing import List

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtcgemm.so")
ARCH = "gfx950"

# (object name, source, extra defines): the host library, the reduction and
# dispatch object, and one GEMM object per input type and layout.
_DT = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}
SOURCES = [("tcgemm", "tcgemm.cpp", []), ("epilogue_kernels", "epilogue_kernels.hip", []),
           ("thin_kernel", "thin_kernel.hip", [])]
for _name, _code in _DT.items():
    for _ta in (0, 1):
        for _tb in (0, 1):
            _lay = ("t" if _ta else "n") + ("t" if _tb else "n")
            SOURCES.append(("gemm_%s_%s" % (_name, _lay), "gemm_inst.hip",
                            ["-DTCG_DT=%d" % _code, "-DTCG_TA=%d" % _ta, "-DTCG_TB=%d" % _tb,
                             "-DTCG_LAUNCHER=tcg_launch_%s_%s" % (_name, _lay)]))

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtcgemm.so")


def _compile(item) -> str:
    name, src, defines = item
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc()] + COMMON + defines + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libtcgemm.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = int(os.environ.get("MAX_JOBS", "0")) or min(16, os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs: List[str] = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
