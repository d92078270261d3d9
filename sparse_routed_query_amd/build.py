"""Build libgqe.so (HIP, gfx950) in-tree with hipcc.

Each source compiles to an object in ``_build/`` in parallel, then one link
step writes ``sparse_routed_query_amd/libgqe.so``; the benchmark's calibration
kernels (``csrc/calib.hip``) link separately into ``libgqe_calib.so``.  Run as a module
(``python -m sparse_routed_query_amd.build``) or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgqe.so")
# calibration kernels for the benchmark's measured ceilings (not part of the path)
CALIB_SRC = "calib.hip"
CALIB_LIB = os.path.join(HERE, "libgqe_calib.so")
SOURCES = ["gqe_api.cpp", "route.hip", "qproj.hip", "attn_prefill.hip", "attn_decode.hip", "outproj.hip",
           "route_bwd.hip", "attn_bwd.hip", "proj_bwd.hip", "decode_pre.hip", "kvproj.hip"]
ARCH = os.environ.get("GQE_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed-fp32 instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: avoids accumulator-register copies in the softmax
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES + [CALIB_SRC]))
    calib_obj = objs.pop()
    _link([calib_obj], CALIB_LIB)
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
