"""Build libcpla.so (gfx950) in-tree with hipcc.

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instructions disabled, then linked into ``context_state_passing_amd/libcpla.so``
next to this file; the benchmark's attainable-peak probes (``csrc/peaks.hip``)
go into ``libcpla_peaks.so`` beside it. ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcpla.so")
PEAKS_LIB = os.path.join(PKG, "libcpla_peaks.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["abi.hip", "fwd.hip", "bwd.hip", "scan.hip", "ssd.hip", "delta.hip", "decay_check.hip", "metadata.cpp"]
PEAKS_SOURCES = ["peaks.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


# The peak probes' MFMA loops keep their accumulators in VGPRs: left to itself the
# compiler places them in AGPRs and copies them back and forth every iteration.
EXTRA_FLAGS = {"peaks.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stderr[-8000:]}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{res.stderr[-8000:]}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
