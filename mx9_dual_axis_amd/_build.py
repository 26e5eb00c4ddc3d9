"""Compile the HIP kernels and the C ABI into ``libmxq.so`` (gfx950 only), and
the benchmark's measurement helpers into ``libmxq_roof.so``."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxq.so")
ROOF_LIB = os.path.join(HERE, "libmxq_roof.so")
SOURCES = ["dual_axis.hip", "mx9.hip", "mx9_layouts.hip", "mx_gemm.hip", "scale_layout.hip", "mxq_abi.cpp"]
ROOF_SOURCES = ["roof.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions are generated (they are not trusted on this target)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose: bool):
    if verbose:
        print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _link(sources, out, objdir, verbose):
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(6, len(cmds))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    _link(SOURCES, LIB, objdir, verbose)
    _link(ROOF_SOURCES, ROOF_LIB, objdir, verbose)
    return LIB


if __name__ == "__main__":
    build()
