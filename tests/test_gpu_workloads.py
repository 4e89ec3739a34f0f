"""The five workloads at full size, through the same entry points and launch
configurations the benchmark times, against the CPU oracle.

Decode-type workloads (M <= 16) are checked on every output element.  The
M = 512 prefill chunk is checked on 256 whole output columns plus 8 whole
output rows (sampled with a fixed seed): the oracle computes those elements
one by one at full K.
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_parity, run

pytestmark = pytest.mark.gpu


def cases(name):
    return synth.workload_cases(name)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_tiny(kind):
    (c,) = cases("tiny")
    y = run(kind, c.matrix.codes, c.matrix.scales, c.matrix.g, c.x)
    assert_parity(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, y)


@pytest.mark.parametrize("name", ["dec", "mtp"])
@pytest.mark.parametrize("mat", ["gate_up", "down"])
def test_decode_and_verify(name, mat):
    (c,) = synth.workload_cases(name, only=[mat])
    y = run("gemv", c.matrix.codes, c.matrix.scales, c.matrix.g, c.x)
    worst = assert_parity(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, y)
    print(f"{name}/{mat}: worst |y-y_ref|/S = {worst:.3g}")


@pytest.mark.parametrize("mat", ["qkv", "gate_up"])
def test_prefill_chunk(mat):
    (c,) = synth.workload_cases("pre", only=[mat])
    y = run("gemm", c.matrix.codes, c.matrix.scales, c.matrix.g, c.x)
    rng = np.random.default_rng(31)
    cols = np.sort(rng.choice(c.N, 256, replace=False))
    rows = np.sort(rng.choice(c.M, 8, replace=False))
    w1 = assert_parity(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, y, rows=cols)
    w2 = assert_parity(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, y, xrows=rows)
    assert np.isfinite(y).all()
    print(f"pre/{mat}: worst |y-y_ref|/S = {max(w1, w2):.3g}")


@pytest.mark.parametrize("mat", ["lm_head", "up_4b", "down_4b"])
def test_lm_head_and_4b(mat):
    (c,) = synth.workload_cases("lmh", only=[mat])
    y = run("gemv", c.matrix.codes, c.matrix.scales, c.matrix.g, c.x)
    worst = assert_parity(c.matrix.codes, c.matrix.scales, c.matrix.g, c.x, y)
    print(f"lmh/{mat}: worst |y-y_ref|/S = {worst:.3g}")
