"""Compile the HIP library libw8inv.so in-tree for gfx950 (hipcc; no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw8inv.so")
# calibration kernels (include/w8calib.h): a separate library, outside the decode path
CALIB_LIB = os.path.join(PKG, "libw8calib.so")
CALIB_SOURCES = ["w8calib.hip"]

SOURCES = ["w8inv_api.hip", "w8inv_gemm.hip", "w8inv_logprob.hip", "w8inv_glue.hip", "w8inv_pack.hip",
           "w8inv_argmax.hip", "w8inv_kslice.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # one IEEE operation per + - * / ; fused operations only where written as fma
    "-ffp-contract=off",
    # keep fp32 subnormals (fp16/fp64 ones are kept by default)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def compile_source(path: str, obj: str, include_dir: str = CSRC) -> str:
    """hipcc -c of one source with the library's flags (`include_dir` holds its private headers)."""
    flags = [f if f != CSRC else include_dir for f in FLAGS]
    r = subprocess.run([HIPCC, *flags, "-c", path, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {path}")
    return obj


def _compile(src: str) -> str:
    return compile_source(os.path.join(CSRC, src), os.path.join(BUILD, src.replace(".hip", ".o")))


def link_objects(objs: list, lib: str) -> None:
    _link(objs, lib)


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, lib)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(CALIB_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
