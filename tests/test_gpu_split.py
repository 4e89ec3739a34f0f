"""The stream-K GEMV's unit split at its edges, against the CPU oracle on every
output.

The launcher deals the units (row tile t, k-tile c) out to workgroups and,
inside a workgroup, to waves, from a split the host computes per range kind
(full K ranges and a shorter last one); the staging of the activations maps
group indices to rows with a fixed-point reciprocal; and the finish finds
the waves that share a row tile from their ranges.  These shapes (on a
256-CU device) put each of those at an edge:

* (1, 16, 128): one unit, one workgroup of one wave;
* (3, 48, 256): three row tiles of two units, one workgroup per tile and
  fewer units than waves;
* (1, 4096, 1152): 2304 units over 256 workgroups, nine each: one wave of
  each workgroup streams two units, the rest one, every row tile split
  between waves and workgroups;
* (2, 4112, 1280): 257 row tiles over 256 workgroups: ten workgroups take
  one unit more than the others, and their waves split 11 units;
* (5, 8192, 640): 2560 units, exactly ten per workgroup;
* (7, 1600, 17168): K = 17168 is 134 whole k-tiles and a 16-wide ragged
  one; its activations need K ranges, and the last range is shorter than
  the others (the second split kind), with two rows per exchange word;
* (16, 272, 9232): 73 k-tiles (ragged) in four ranges of 19, 19, 19 and 16;
* (12, 4352, 3088): 272 row tiles of 25 k-tiles (ragged), three rows a lane;
* (9, 3000, 6160): 188 row tiles (ragged N) of 49 k-tiles (ragged K).

Each runs the plain GEMV (y checked everywhere), the fused gate/up variant
where N is a multiple of 16 (h checked everywhere) and the argmax variant
(index and value checked), twice each for bitwise repeatability.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_parity, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16, 128), (3, 48, 256), (1, 4096, 1152), (2, 4112, 1280), (5, 8192, 640),
          (7, 1600, 17168), (16, 272, 9232), (12, 4352, 3088), (9, 3000, 6160)]


def gemv(packed, g, x, N, K):
    M = x.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q4().q4proj_gemv(packed[0], packed[1], g, to_dev_x(x), y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_split_edges(M, N, K):
    m = q4()
    w = synth.nvfp4_normal_matrix(300 + M, 5, N, K)
    x = synth.x_bf16(300 + M, 6, M, K)
    packed = pack(w.codes, w.scales, N, K)

    note(f"gemv split edges M={M} N={N} K={K}")
    y = gemv(packed, w.g, x, N, K)
    assert_parity(w.codes, w.scales, w.g, x, y)
    assert np.array_equal(y.view(np.uint32), gemv(packed, w.g, x, N, K).view(np.uint32))

    if N % 16 == 0:
        F = N // 2
        note(f"gemv_silu_mul split edges M={M} F={F} K={K}")
        h = torch.full((M, F), -1, dtype=torch.int16, device=DEV)
        m.q4proj_gemv_silu_mul(packed[0], packed[1], w.g, to_dev_x(x), h, M, F, K)
        torch.cuda.synchronize()
        hh = h.cpu().numpy().view(np.uint16)
        href, bound = oracle.silu_mul_cols(w.codes, w.scales, w.g, x, F)
        bad, worst = oracle.check_bf16(href, bound, hh)
        assert bad == 0, f"{bad} outputs outside the allowance (worst ratio {worst:.3g})"

    note(f"gemv_argmax split edges M={M} N={N} K={K}")
    val = torch.empty(M, dtype=torch.float32, device=DEV)
    idx = torch.empty(M, dtype=torch.int64, device=DEV)
    m.q4proj_gemv_argmax(packed[0], packed[1], w.g, to_dev_x(x), None, val, idx, M, N, K)
    torch.cuda.synchronize()
    yr, S = oracle.proj(w.codes, w.scales, w.g, x)
    assert oracle.argmax_check(yr, S, idx.cpu().numpy(), val.cpu().numpy()) == 0
    # the argmax of the GEMV's own logits (the same sums), first index on ties
    ii = idx.cpu().numpy()
    assert np.array_equal(ii, np.argmax(y, axis=1))
    assert np.array_equal(val.cpu().numpy().view(np.uint32), y[np.arange(M), ii].view(np.uint32))
