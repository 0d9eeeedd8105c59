"""Build libtplinear.so (gfx950 only) in-tree with hipcc.

    python -m tensor_linear_amd.build

Every device source is compiled with packed-fp32 instructions turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtplinear.so")
# Shader-clock probe the bench runs next to a GEMM (a library of its own, not
# part of the tensor-parallel ABI).
CLOCK_LIB = os.path.join(HERE, "libtplclock.so")
CLOCK_SOURCE = "clock_probe.hip"

SOURCES = ["tplinear.cpp", "device.cpp", "gemm_tile.hip", "gemm_skinny.hip", "gemm_generic.hip",
           "shard_fold.hip", "embedding.hip", "gemm_rowfold.hip", "gemm_narrow.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [CLOCK_SOURCE]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], CLOCK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
