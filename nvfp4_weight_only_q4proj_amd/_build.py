"""Build libq4proj.so (gfx950 only) in-tree with hipcc.

    python nvfp4_weight_only_q4proj_amd/_build.py

(run by path: importing the package needs the library it builds)

Every HIP source is compiled with packed-FP32 instruction selection turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns
that it does not know the feature, which is expected.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libq4proj.so")

HIP_SOURCES = ["q4p_pack.hip", "q4p_gemv.hip", "q4p_gemm.hip", "q4p_quant.hip"]
HOST_SOURCES = ["q4p_api.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-fno-gpu-flush-denormals-to-zero"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, out: str = LIB) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    hipcc = _hipcc()
    for src in HIP_SOURCES + HOST_SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
