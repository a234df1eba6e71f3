"""Build libopq.so in-tree with hipcc for gfx950.

    python -m w4a16_linear_amd.build [-v]

HIP sources are compiled for gfx950 only, without fast-math (the quantizer
relies on correctly rounded binary32 division and kept subnormals) and with
packed fp32 instructions disabled.  Host-only C++ (the ABI layer and the
binary128 table code, which needs libquadmath) is compiled with g++.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libopq.so")
# the benchmark's streaming-ceiling kernel, a library of its own
CEILING_LIB = os.path.join(HERE, "libopq_ceiling.so")

SOURCES = ["opq_api.cpp", "tables.cpp", "quantize.hip", "dequantize.hip", "linear.hip"]
CEILING_SOURCES = ["stream_ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found at {path}")
    return path


def hip_flags() -> list:
    """hipcc flags of every HIP source (gfx950, no fast-math, packed fp32 off)."""
    return [f"--offload-arch={ARCH}", "-x", "hip", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def device_asm(src: str) -> str:
    """gfx950 assembly of one HIP source, compiled as the library is (the kernel
    metadata at its end gives each kernel's registers and scratch)."""
    cmd = [hipcc()] + hip_flags() + ["--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stderr}")
    return r.stdout


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
    if src.endswith(".hip"):
        cmd = [hipcc()] + hip_flags()
    else:
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
        cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
        cmd = [cxx, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include")] + common
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def _link(objs, lib: str, libs, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + libs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libopq.so and libopq_ceiling.so; returns the
    path of libopq.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, ["-lquadmath"], verbose)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
