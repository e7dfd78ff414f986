"""Compile the HIP kernels and the C ABI into libspmla.so (gfx950 only).

Usage: python -m sparse_long_context_int8_amd.build   (or call build()).
The library is written next to this file; it is a build product and is not
kept in version control.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libspmla.so")
SOURCES = ["api.cpp", "plan.cpp", "indexer.hip", "topk.hip", "attn.hip", "compress.hip", "noalloc.hip"]
# Measurement kernel of the benchmark (not part of the layer), its own library.
CEILING_SOURCES = ["ceiling.hip"]
CEILING_LIB_PATH = os.path.join(HERE, "libspmla_ceiling.so")
ARCH = "gfx950"
# Per-source code generation options. The int8 indexer kernels consume every
# matrix-core result with vector ops at once; the VGPR form of the MFMA
# instructions saves an accumulator-register read per result element.
EXTRA_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libspmla.so")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Keep hipcc from emitting packed fp32 VALU ops (v_pk_*_f32).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        "-Wall",
        "-Wno-unused-function",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Builds libspmla.so (the layer) and libspmla_ceiling.so (the gather
    ceiling measurement kernel the benchmark reports against)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {CEILING_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
