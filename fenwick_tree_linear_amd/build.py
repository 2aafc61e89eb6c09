"""Builds libllattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m fenwick_tree_linear_amd.build

Each translation unit is compiled by hipcc in parallel, then linked into
``fenwick_tree_linear_amd/libllattn.so``.  Packed fp32 vector instructions are
switched off for every device compilation.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libllattn.so")
OBJ_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "chunk_attn.hip", "fenwick_scan.hip", "decode_step.hip", "gdn.hip", "lambda_mlp.hip", "prior_read.hip", "ccq.hip", "bwd_native.hip", "pad.hip"]
ARCH = os.environ.get("LLATTN_ARCH", "gfx950")

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
    "-Wno-unused-function",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [_hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _check_no_undefined_kernels(lib: str) -> None:
    """A kernel whose host stub the compiler did not emit links silently and
    only fails when the library is loaded: refuse such a library here."""
    readelf = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-readelf")
    r = subprocess.run([readelf, "--dyn-syms", "-W", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-readelf failed on {lib}:\n{r.stderr}")
    missing = [line.split()[-1] for line in r.stdout.splitlines() if " UND " in line and "llattn" in line]
    if missing:
        raise RuntimeError("undefined kernel symbols in the built library: " + ", ".join(missing))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    _check_no_undefined_kernels(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
