"""The C ABI from plain C: tests/c_abi/abi_consumer.c allocates device memory
with the HIP runtime, packs a seeded weight, runs q4proj_gemv and q4proj_gemm
on its own stream, checks them against the CPU oracle, checks the documented
rejections (M > 16, a null output, K % 16 != 0, a short workspace) and the
pack/unpack round trip; then the greedy argmax, the fused gate/up pack from
two separate weights with both fused projections, and the quantizer (bit for
bit), each against the oracle.  It is loaded as a shared library and called
in-process (no Python objects cross the ABI)."""
import ctypes
import os

import pytest

from gpu_util import note

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_plain_c_consumer(capfd):
    lib_path = os.path.join(HERE, "c_abi", "libabi_consumer.so")
    # built by __graft_entry__.build(); a process that uses the GPU starts no
    # compiler
    assert os.path.exists(lib_path), f"{lib_path} missing: run __graft_entry__.build() first"
    note("plain C consumer of the C ABI (gemv M=3, gemm M=40, N=300, K=1040; argmax, "
         "pack_gate_up + silu_mul, quantize)")
    lib = ctypes.CDLL(lib_path)
    lib.abi_consumer_run.restype = ctypes.c_int
    rc = lib.abi_consumer_run()
    out, err = capfd.readouterr()
    print(out, err)
    assert rc == 0, err
    assert "all checks passed" in out
