"""q4proj_gemv / q4proj_gemm against the CPU oracle on small and ragged shapes.

* every code x scale product, exactly (all 256 e4m3 encodings x 16 codes);
* one-hot activations return exactly the dequantised column;
* brute-force tiny shapes within tolerance (and far inside it);
* ragged M, N, K spanning several tiles plus a tail;
* invariants: repeatability, permutation, g scaling and zero input bitwise;
  sign bitwise for gemv, within 1e-6 * S for gemm.
"""
import numpy as np
import pytest
import torch

import oracle
import pins
import synth
from gpu_util import (DEV, assert_parity, bits, note, oracle_fp32, pack, project, q4, run,
                      to_dev_x)

pytestmark = pytest.mark.gpu

KINDS = ["gemv", "gemm", "gemm_bf16"]     # gemm: fp16 operands, gemm_bf16: without a workspace


def same_values(a, b):
    """Value-exact equality with NaN positions matching (-0 == +0)."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb])


def all_products_weight():
    """N = 256 rows, row n uses scale byte n everywhere; element k has code k % 16."""
    N, K = 256, 256
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    code = (np.arange(K) % 16).astype(np.uint8)
    codes = np.repeat((code[0::2] | (code[1::2] << 4)).astype(np.uint8)[None, :], N, axis=0)
    return codes, scales


def one_hot(ks, K):
    x = np.zeros((len(ks), K), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80          # bf16 1.0
    return x


def test_all_code_scale_products_gemm_identity():
    codes, scales = all_products_weight()
    x = one_hot(np.arange(256), 256)             # x = I_256
    y = run("gemm", codes, scales, 1.0, x)
    want = oracle_fp32(codes, scales, 1.0, x)
    assert same_values(y, want)
    # spot values: y[m][n] = e2m1(m % 16) * e4m3(n)
    assert y[2, 0x38] == 1.0 and y[7, 0x7E] == 6 * 448.0 and y[15, 0x01] == -6 * 2.0 ** -9
    assert np.isnan(y[:, 0x7F]).all() and np.isnan(y[:, 0xFF]).all()


def test_all_code_scale_products_gemv_batches():
    codes, scales = all_products_weight()
    packed = pack(codes, scales, 256, 256)
    for b in range(16):
        x = one_hot(16 * b + np.arange(16), 256)
        note(f"gemv all-products batch {b}")
        y = project("gemv", packed, 1.0, x, 256, 256)
        assert same_values(y, oracle_fp32(codes, scales, 1.0, x)), b


@pytest.mark.parametrize("kind", KINDS)
def test_one_hot_returns_dequantised_columns(kind):
    m = synth.nvfp4_normal_matrix(11, 1, 272, 1040)
    rng = np.random.default_rng(2)
    ks = rng.choice(1040, 16, replace=False)
    x = one_hot(ks, 1040)
    y = run(kind, m.codes, m.scales, m.g, x)
    want = oracle_fp32(m.codes, m.scales, m.g, x)   # one rounding of q*s*g to fp32
    assert same_values(y, want)


TINY = [(M, N, K) for M in (1, 2, 7, 16, 33) for N in (1, 16, 17, 64) for K in (16, 32, 48, 256)]


@pytest.mark.parametrize("kind", KINDS)
def test_brute_force_tiny(kind):
    worst = 0.0
    for i, (M, N, K) in enumerate(TINY):
        if kind == "gemv" and M > 16:
            continue
        codes, scales, x = pins.tiny_inputs(M, N, K, 500 + i)
        for g in (1.0, 2.0 ** -10, float(np.float32(3.3e-5))):
            y = run(kind, codes, scales, g, x)
            worst = max(worst, assert_parity(codes, scales, g, x, y))
    print(f"{kind} tiny worst |y-y_ref|/S = {worst:.3g}")


RAGGED = {
    # (7, 4352, 640) .. (12, 5000, 3088) have more row tiles than a 256-CU
    # device has CUs and per-CU ranges that end inside row tiles: their split
    # row tiles are finished across workgroups, for every output row M can
    # hold.  (16, 272, 2000), (12, 130, 9216) and (7, 200, 17408) ..
    # (16, 1000, 32768) cut K into 2, 4, 8, 8, 2 (ragged) and 8 ranges
    # (the launcher's cost estimate picks the count) whose results are
    # joined per output, two rows per word above M = 4.  The last three need
    # more than 8 ranges (a range's activations would not fit in LDS) and run
    # on the split kernel (activation pieces in the register ring): M > 8,
    # M = 1 and M = 3.
    "gemv": [(5, 1000, 1040), (16, 272, 2000), (1, 3, 4112), (7, 33, 144), (3, 4097, 128),
             (12, 130, 9216), (7, 4352, 640), (2, 6000, 272), (16, 4368, 912),
             (12, 5000, 3088), (7, 200, 17408), (16, 272, 16384), (9, 4352, 8320),
             (16, 1000, 32768), (16, 300, 36864), (1, 100, 1048576), (3, 40, 200000)],
    "gemm": [(129, 300, 1040), (513, 100, 272), (1, 17, 5136), (200, 4112, 128),
             (64, 2049, 400), (300, 48, 2000)],
}
RAGGED["gemm_bf16"] = RAGGED["gemm"]


@pytest.mark.parametrize("kind", KINDS)
def test_ragged_shapes(kind):
    for i, (M, N, K) in enumerate(RAGGED[kind]):
        m = synth.nvfp4_normal_matrix(40 + i, 3, N, K)
        x = synth.x_bf16(40 + i, 4, M, K)
        y = run(kind, m.codes, m.scales, m.g, x)
        assert_parity(m.codes, m.scales, m.g, x, y)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemv_every_m(M):
    """Every M of the decode/verify range on two shapes: 4352 x 640 (272 row
    tiles over one workgroup per CU, so row tiles are split between waves and
    between workgroups) and 300 x K with K cut into ranges (four at these
    sizes: the activations of all of K would not fit in LDS, and the joins
    of 300 columns are cheap).  Each M places its rows differently in the
    lanes' output slots (one per lane up to M = 4, two up to M = 8, three or
    four above) and above M = 4 joins two rows per exchange word."""
    for j, (N, K) in enumerate([(4352, 640), (300, 128 * (512 // M + 4))]):
        m = synth.nvfp4_normal_matrix(60 + M, 3 + j, N, K)
        x = synth.x_bf16(60 + M, 4 + j, M, K)
        y = run("gemv", m.codes, m.scales, m.g, x)
        assert_parity(m.codes, m.scales, m.g, x, y)


@pytest.mark.parametrize("M", [1, 129, 200, 383])
def test_gemm_writes_no_row_past_m(M):
    """y is the first M rows of a larger buffer whose other rows hold a
    sentinel: the last 128-row block's rows past M are dropped at the end of
    the output buffer, so the sentinel must survive bit for bit."""
    m = q4()
    N, K = 272, 640
    w = synth.nvfp4_normal_matrix(90 + M, 1, N, K)
    x = synth.x_bf16(90 + M, 2, M, K)
    packed = pack(w.codes, w.scales, N, K)
    big = torch.full((M + 256, N), 12345.0, dtype=torch.float32, device=DEV)
    note(f"gemm guard rows M={M} N={N} K={K}")
    m.q4proj_gemm(packed[0], packed[1], w.g, to_dev_x(x), big[:M], M, N, K)
    torch.cuda.synchronize()
    tail = big[M:].cpu()
    assert bool((tail == 12345.0).all()), "rows past M were written"
    assert_parity(w.codes, w.scales, w.g, x, big[:M].cpu().numpy())


@pytest.mark.parametrize("M,N,K", [(1, 4099, 640), (7, 4352, 17408), (16, 300, 1040)])
def test_gemv_writes_nothing_past_y(M, N, K):
    """y (M x N, ragged N, one and two K ranges) is the start of a larger
    sentinel-filled buffer: nothing after its M*N elements may change."""
    m = q4()
    w = synth.nvfp4_normal_matrix(97 + M, 1, N, K)
    x = synth.x_bf16(97 + M, 2, M, K)
    packed = pack(w.codes, w.scales, N, K)
    big = torch.full((M * N + 4096,), 12345.0, dtype=torch.float32, device=DEV)
    note(f"gemv guard M={M} N={N} K={K}")
    m.q4proj_gemv(packed[0], packed[1], w.g, to_dev_x(x), big[:M * N], M, N, K)
    torch.cuda.synchronize()
    assert bool((big[M * N:].cpu() == 12345.0).all()), "elements past y were written"
    assert_parity(w.codes, w.scales, w.g, x, big[:M * N].cpu().numpy().reshape(M, N))


@pytest.mark.parametrize("kind", KINDS)
def test_nan_and_zero_scales(kind):
    codes, scales, x = pins.tiny_inputs(7, 40, 96, 77)
    scales[3, 2] = 0x7F
    scales[20, :] = 0xFF
    scales[9, :] = 0x00            # all-zero row
    scales[11, 1] = 0x80           # -0 scale block
    y = run(kind, codes, scales, 0.5, x)
    assert np.isnan(y[:, [3, 20]]).all()
    assert (y[:, 9] == 0).all()
    assert np.isfinite(np.delete(y, [3, 20], axis=1)).all()
    assert_parity(codes, scales, 0.5, x, y)


@pytest.mark.parametrize("kind", KINDS)
def test_invariants_bitwise(kind):
    M = 7 if kind == "gemv" else 40
    N, K = 100, 656
    w = synth.nvfp4_normal_matrix(8, 1, N, K)
    x = synth.x_bf16(8, 2, M, K)
    packed = pack(w.codes, w.scales, N, K)
    y = project(kind, packed, w.g, x, N, K)
    assert_parity(w.codes, w.scales, w.g, x, y)
    # repeatability: same bits on every call
    for _ in range(3):
        assert np.array_equal(bits(project(kind, packed, w.g, x, N, K)), bits(y))
    # y(-x) = -y(x): bitwise for gemv, whose matrix-core sums are 16 exact
    # products started from zero and whose scale/accumulate steps are
    # round-to-nearest fmas.  The bf16 MFMA's long accumulation into a running
    # fp32 sum is not sign-symmetric in its last bits on gfx950 (measured: 2 of
    # 4000 outputs off by 2-3 ulp), so gemm is held to 1e-6 * S instead.
    yn = project(kind, packed, w.g, x ^ np.uint16(0x8000), N, K)
    if kind == "gemv":
        assert np.array_equal(bits(yn), bits(-y))
    else:
        _, S = oracle.proj(w.codes, w.scales, w.g, x)
        assert (np.abs(yn.astype(np.float64) + y) <= 1e-6 * S).all()
    # g -> 2g doubles y
    y2 = project(kind, packed, 2 * w.g, x, N, K)
    assert np.array_equal(bits(y2), bits(2 * y))
    # x = 0 gives +0 everywhere
    y0 = project(kind, packed, w.g, np.zeros_like(x), N, K)
    assert (y0 == 0).all()
    # permuting 16-row tiles of W permutes y's columns (each output only
    # depends on its own weight row)
    perm_tiles = np.random.default_rng(3).permutation(-(-N // 16) - 1)   # keep the ragged tile last
    perm = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in perm_tiles] +
                          [np.arange(16 * len(perm_tiles), N)])
    yp = project(kind, pack(w.codes[perm], w.scales[perm], N, K), w.g, x, N, K)
    assert np.array_equal(bits(yp), bits(y[:, perm]))


def test_gemv_and_gemm_agree_within_tolerance():
    N, K, M = 512, 3072, 16
    w = synth.nvfp4_normal_matrix(9, 1, N, K)
    x = synth.x_bf16(9, 2, M, K)
    packed = pack(w.codes, w.scales, N, K)
    yv = project("gemv", packed, w.g, x, N, K)
    ym = project("gemm", packed, w.g, x, N, K)
    assert_parity(w.codes, w.scales, w.g, x, yv)
    assert_parity(w.codes, w.scales, w.g, x, ym)


def test_gemv_rejects_m_above_16():
    m = q4()
    w = synth.nvfp4_normal_matrix(1, 1, 16, 128)
    packed = pack(w.codes, w.scales, 16, 128)
    x = to_dev_x(np.zeros((17, 128), np.uint16))
    y = torch.empty((17, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(m.Q4ProjError) as e:
        m.q4proj_gemv(packed[0], packed[1], 1.0, x, y, 17, 16, 128)
    assert e.value.status == m.EUNSUPPORTED
