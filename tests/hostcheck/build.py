"""Build the CPU check of the library's host front under AddressSanitizer and
UndefinedBehaviorSanitizer: nvfp4_weight_only_q4proj_amd/csrc/q4p_api.cpp
compiled with g++ against the stand-in HIP header in this directory, linked
with the recording stubs and the C driver into one executable,
tests/hostcheck/hostcheck.  CPU code only: no HIP compiler, no GPU code.
Test infrastructure: called by __graft_entry__.build().
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "nvfp4_weight_only_q4proj_amd", "csrc")
OUT = os.path.join(HERE, "hostcheck")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build(out: str = OUT, verbose: bool = False) -> str:
    inc = ["-I", HERE, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        steps = [
            ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", *SAN, *inc, "-c",
             os.path.join(CSRC, "q4p_api.cpp"), "-o", os.path.join(tmp, "api.o")],
            ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", *SAN, *inc, "-c",
             os.path.join(HERE, "stubs.cpp"), "-o", os.path.join(tmp, "stubs.o")],
            ["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", *SAN, *inc, "-c",
             os.path.join(HERE, "hostcheck.c"), "-o", os.path.join(tmp, "hostcheck.o")],
        ]
        for cmd in steps:
            if verbose:
                print(" ".join(cmd))
            subprocess.run(cmd, check=True)
            objs.append(cmd[-1])
        link = ["g++", *SAN, "-o", out + ".tmp", *objs, "-lm"]
        if verbose:
            print(" ".join(link))
        subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
