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


# The host layer (argument validation, launch planning) with AddressSanitizer, for the CPU tests of
# the C ABI: w8inv_api.hip built with ASan on its host side only (each -fsanitize= after -Xarch_host),
# linked with the product's other objects; loaded with the ASan runtime preloaded.
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libw8inv_hostasan.so")
HOST_ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang ASan runtime shared library of the ROCm toolchain ("" if absent)."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else ""


def build_host_asan() -> str:
    os.makedirs(ASAN_DIR, exist_ok=True)
    api = "w8inv_api.hip"
    obj = os.path.join(ASAN_DIR, api.replace(".hip", ".o"))
    r = subprocess.run([HIPCC, *FLAGS, *HOST_ASAN_FLAGS, "-c", os.path.join(CSRC, api), "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on the host-ASan build of " + api)
    others = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES if s != api]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        others = [_compile(s) for s in SOURCES if s != api]
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        obj, *others, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed (host-ASan library)")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build())
