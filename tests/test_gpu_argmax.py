"""q4proj_gemv_argmax (the lm-head GEMV with a fused greedy argmax).

* the decision matches torch.argmax over the same kernel's fp32 logits
  exactly (first maximum, NaN largest), and the value is that logit bit for
  bit; the logits equal q4proj_gemv's bit for bit; with y = NULL the result
  is the same;
* against the oracle (several indices can be correct within tolerance):
  small and ragged shapes, the full lm-head at M = 1 and M = 4, and a shape
  with two K ranges at M = 16;
* exact ties (one-hot activations over duplicated weight rows) pick the
  lowest index; NaN rows pick their first NaN; all-zero and all-negative
  logits; repeated calls on one workspace.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def run_argmax(packed, g, x, N, K, with_y=True, workspace=None):
    m = q4()
    M = x.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV) if with_y else None
    val = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
    idx = torch.full((M,), -1, dtype=torch.int64, device=DEV)
    m.q4proj_gemv_argmax(packed[0], packed[1], g, to_dev_x(x), y, val, idx, M, N, K,
                         workspace=workspace)
    torch.cuda.synchronize()
    return (None if y is None else y.cpu()), val.cpu(), idx.cpu()


def assert_self_consistent(y, val, idx):
    want = torch.argmax(y, dim=1)
    assert torch.equal(idx, want), (idx, want)
    picked = y[torch.arange(y.shape[0]), idx]
    nan = torch.isnan(picked)
    assert torch.equal(torch.isnan(val), nan)
    assert torch.equal(val[~nan].view(torch.int32), picked[~nan].view(torch.int32))


def check(mat, x, with_oracle=True):
    N, K = mat.codes.shape[0], mat.codes.shape[1] * 2
    packed = pack(mat.codes, mat.scales, N, K)
    note(f"gemv_argmax M={x.shape[0]} N={N} K={K}")
    y, val, idx = run_argmax(packed, mat.g, x, N, K)
    assert_self_consistent(y, val, idx)
    _, val2, idx2 = run_argmax(packed, mat.g, x, N, K, with_y=False)
    assert torch.equal(idx2, idx) and torch.equal(val2.view(torch.int32), val.view(torch.int32))
    if with_oracle:
        yr, S = oracle.proj(mat.codes, mat.scales, mat.g, x)
        assert oracle.argmax_check(yr, S, idx.numpy(), val.numpy()) == 0
    return packed, y, val, idx


SMALL = [(M, N, K) for M in (1, 2, 3, 7, 16) for N in (1, 17, 300, 4099) for K in (16, 208, 1040)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes(M, N, K):
    mat = synth.nvfp4_normal_matrix(110 + M, 1, N, K)
    x = synth.x_bf16(110, N % 97, M, K)
    check(mat, x)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_every_m(M):
    """Every M from 1 to 16 over 4352 x 640 (row tiles split between waves and
    workgroups) and 300 x K with two K ranges."""
    for j, (N, K) in enumerate([(4352, 640), (300, 128 * (512 // M + 4))]):
        mat = synth.nvfp4_normal_matrix(130 + M, 1 + j, N, K)
        x = synth.x_bf16(130 + j, M, M, K)
        check(mat, x)


def test_logits_equal_plain_gemv():
    mat = synth.nvfp4_normal_matrix(120, 1, 20000, 3072)
    x = synth.x_bf16(120, 1, 5, 3072)
    packed, y, _, _ = check(mat, x, with_oracle=False)
    ref = torch.empty((5, 20000), dtype=torch.float32, device=DEV)
    q4().q4proj_gemv(packed[0], packed[1], mat.g, to_dev_x(x), ref, 5, 20000, 3072)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), ref.cpu().view(torch.int32))


@pytest.mark.parametrize("M", [1, 4])
def test_lm_head_full_size(M):
    (c,) = synth.workload_cases("lmh", only=["lm_head"])
    x = c.x if M == 1 else synth.x_bf16(4, 20 + M, M, c.K)
    check(c.matrix, x)


def test_two_k_ranges():
    # M = 16 at K = 5120: 160 KB of activations, cut into two K ranges
    mat = synth.nvfp4_normal_matrix(130, 1, 32768, 5120)
    x = synth.x_bf16(130, 1, 16, 5120)
    check(mat, x)


def test_exact_ties_pick_the_lowest_index():
    N, K, M = 3000, 256, 4
    mat = synth.nvfp4_normal_matrix(140, 1, N, K)
    codes, scales = mat.codes.copy(), mat.scales.copy()
    # row 41: code 6.0 (0x7) at every k and the top scale, the largest value
    # any row can reach; rows 2999, 1500, 777 and 40 copy it, so with one-hot
    # activations their logits are the same single product, bit for bit
    codes[41] = 0x77
    scales[41] = 0x7E
    for r in (2999, 1500, 777, 40):
        codes[r], scales[r] = codes[41], scales[41]
    codes[:40] = 0                                       # nothing below row 40 reaches it
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), [0, 17, 100, 255]] = 0x3F80          # one-hot rows (bf16 1.0)
    packed = pack(codes, scales, N, K)
    note("gemv_argmax exact ties")
    y, val, idx = run_argmax(packed, mat.g, x, N, K)
    assert (idx == 40).all(), idx
    assert_self_consistent(y, val, idx)


def test_nan_rows_zero_and_negative_logits():
    N, K = 2048, 512
    mat = synth.nvfp4_normal_matrix(150, 1, N, K)
    scales = mat.scales.copy()
    scales[1234, 5] = 0x7F                                # NaN scale: logits of row 1234
    scales[333, 0] = 0xFF                                 # and row 333 are NaN
    packed = pack(mat.codes, scales, N, K)
    x = synth.x_bf16(150, 1, 2, K)
    note("gemv_argmax NaN rows")
    y, val, idx = run_argmax(packed, mat.g, x, N, K)
    assert (idx == 333).all() and torch.isnan(val).all()
    yr, S = oracle.proj(mat.codes, scales, mat.g, x)
    assert oracle.argmax_check(yr, S, idx.numpy(), val.numpy()) == 0
    # all-zero activations: every logit is +-0, the first column wins
    packed = pack(mat.codes, mat.scales, N, K)
    y, val, idx = run_argmax(packed, mat.g, np.zeros((3, K), np.uint16), N, K)
    assert (idx == 0).all() and (val == 0).all()
    # all logits negative: codes all -6 (0xF), x positive
    codes = np.full_like(mat.codes, 0xFF)
    packed = pack(codes, mat.scales, N, K)
    xp = synth.x_bf16(151, 1, 2, K) & np.uint16(0x7FFF)             # |x|: sign bits cleared
    y, val, idx = run_argmax(packed, mat.g, xp, N, K)
    assert (val < 0).all()
    assert_self_consistent(y, val, idx)
    yr, S = oracle.proj(codes, mat.scales, mat.g, xp)
    assert oracle.argmax_check(yr, S, idx.numpy(), val.numpy()) == 0


def test_repeated_calls_one_workspace():
    mat = synth.nvfp4_normal_matrix(160, 1, 50000, 2048)
    x = synth.x_bf16(160, 1, 3, 2048)
    N, K = 50000, 2048
    packed = pack(mat.codes, mat.scales, N, K)
    ws = torch.zeros(q4().q4proj_argmax_workspace_bytes(3, N, K), dtype=torch.uint8, device=DEV)
    note("gemv_argmax repeated calls")
    first = run_argmax(packed, mat.g, x, N, K, with_y=False, workspace=ws)
    for _ in range(5):
        again = run_argmax(packed, mat.g, x, N, K, with_y=False, workspace=ws)
        assert torch.equal(again[2], first[2])
        assert torch.equal(again[1].view(torch.int32), first[1].view(torch.int32))
    assert int(torch.count_nonzero(ws)) == 0
    # a smaller call on the same workspace
    x1 = x[:1]
    _, val, idx = run_argmax(packed, mat.g, x1, N, K, with_y=False, workspace=ws)
    assert idx[0] == first[2][0]
    assert int(torch.count_nonzero(ws)) == 0
