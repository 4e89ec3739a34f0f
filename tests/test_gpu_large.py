"""The prefill GEMM past 1 GiB of activations or of packed codes, where the
launcher splits the problem into several launches over row ranges or weight
tile ranges (32-bit buffer offsets), against the CPU oracle on the outputs
on both sides of each split; and with output rows so long that a launch's
outputs pass 2 GiB, where the kernel stores with plain addresses instead of
32-bit buffer offsets (plain and fused gate/up)."""
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


def test_gemm_outputs_past_two_gib_of_offsets():
    # rows of 4.2M fp32 outputs (16.8 MB): the launch's rows plus one block of
    # 128 rows pass 2 GiB, so y is written with plain addresses and per-row
    # tests instead of 32-bit buffer offsets
    M, N, K = 2, 4_200_000, 16
    m = synth.uniform_code_matrix(62, N, K, name="wide")
    x = synth.x_bf16(62, 4, M, K)
    y = run("gemm", m.codes, m.scales, m.g, x)
    cols = np.array([0, 1, 15, 16, 2_097_151, 2_097_152, 4_199_983, 4_199_999])
    assert_parity(m.codes, m.scales, m.g, x, y, rows=cols)
    assert np.isfinite(y).all()


def test_gemm_silu_outputs_past_two_gib_of_offsets():
    # the fused gate/up GEMM with h rows of 8.4M bf16 (16.8 MB): plain-address
    # stores as above
    import oracle
    from gpu_util import DEV, pack, q4, to_dev_x
    import torch
    M, F, K = 1, 8_400_000, 16
    mat = synth.uniform_code_matrix(63, 2 * F, K, name="wide")
    x = synth.x_bf16(63, 4, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    h = torch.full((M, F), -1, dtype=torch.int16, device=DEV)
    q4().q4proj_gemm_silu_mul(packed[0], packed[1], mat.g, to_dev_x(x), h, M, F, K)
    torch.cuda.synchronize()
    hg = h.cpu().numpy().view(np.uint16)
    cols = np.array([0, 7, 8, 4_194_303, 4_194_304, 8_399_992, 8_399_999])
    href, bound = oracle.silu_mul_cols(mat.codes, mat.scales, mat.g, x, F, cols=cols)
    bad, _ = oracle.check_bf16(href, bound, hg[:, cols])
    assert bad == 0
    assert (hg != 0xFFFF).all()
