"""The prefill GEMM past 1 GiB of activations or of packed codes, where the
launcher splits the problem into several launches over row ranges or weight
tile ranges (32-bit buffer offsets), against the CPU oracle on the outputs
on both sides of each split."""
import numpy as np
import pytest

import synth
from gpu_util import assert_parity, run

pytestmark = pytest.mark.gpu


def test_gemm_rows_past_one_gib_of_activations():
    # 65600 x 8192 bf16 = 1.07 GB: rows 0..65535 in one launch, the rest in
    # a second one
    M, N, K = 65600, 48, 8192
    m = synth.nvfp4_normal_matrix(60, 3, N, K)
    x = synth.x_bf16(60, 4, M, K)
    y = run("gemm", m.codes, m.scales, m.g, x)
    rows = np.array([0, 1, 127, 65535, 65536, 65537, 65599])
    assert_parity(m.codes, m.scales, m.g, x, y, xrows=rows)
    assert np.isfinite(y).all()


def test_gemm_tiles_past_one_gib_of_codes():
    # 16400 x 131072 weights: 1025 row tiles x 1024 k-tiles x 1 KB of packed
    # codes; tiles 0..1023 in one launch, the last one in a second
    M, N, K = 2, 16400, 131072
    m = synth.uniform_code_matrix(61, N, K, name="big")
    x = synth.x_bf16(61, 4, M, K)
    y = run("gemm", m.codes, m.scales, m.g, x)
    cols = np.array([0, 15, 16, 8191, 16367, 16383, 16384, 16390, 16399])
    assert_parity(m.codes, m.scales, m.g, x, y, rows=cols)
    assert np.isfinite(y).all()
