"""Build the plain C consumer of the C ABI (tests/c_abi/abi_consumer.c) as a
shared library with one entry point, abi_consumer_run().

It links the product library (libq4proj.so), the CPU oracle and the seeded
input generators, plus the HIP runtime for its own device allocations, with
run paths relative to the binary so the tree can move.  Test infrastructure:
called by __graft_entry__.build() only (the GPU test that runs the consumer
requires it to be built already).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.c")
OUT = os.path.join(HERE, "libabi_consumer.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = OUT, verbose: bool = False) -> str:
    libdirs = [os.path.join(ROOT, "nvfp4_weight_only_q4proj_amd"), os.path.join(ROOT, "oracle"),
               os.path.join(ROOT, "synth")]
    for d, name in zip(libdirs, ("libq4proj.so", "liboracle.so", "libsynth.so")):
        if not os.path.exists(os.path.join(d, name)):
            raise FileNotFoundError(f"{name} is not built (run __graft_entry__.build())")
    rpath = ":".join(["$ORIGIN/../../nvfp4_weight_only_q4proj_amd", "$ORIGIN/../../oracle",
                      "$ORIGIN/../../synth", os.path.join(ROCM, "lib")])
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           SRC, "-o", out + ".tmp"]
    for d in libdirs:
        cmd += ["-L", d]
    cmd += ["-lq4proj", "-loracle", "-lsynth", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath," + rpath]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
