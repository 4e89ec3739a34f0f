"""q4proj_gemv_silu_mul and q4proj_gemm_silu_mul (fused gate/up projection +
silu(gate)*up, bf16 out) against the CPU oracle.

* small and ragged shapes on every output, including shapes whose waves hold
  many whole tiles, tiles shared by waves and workgroups (pairs exchanged in
  one word), and two K ranges (pairs joined in one word);
* the full decode shape (M = 1, F = 17408, K = 5120) and the verify shapes
  M = 7 and M = 16 on sampled outputs;
* against the unfused path: q4proj_gemv on the same packed weight gives the
  gate and up values; silu(gate)*up of those, rounded once to bf16 in fp64,
  is what the epilogue must return up to its own fp32 evaluation;
* repeatability (bitwise), a workspace left zero-filled, NaN scales.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def fused_matrix(seed, F, K):
    return synth.nvfp4_normal_matrix(seed, 1, 2 * F, K)


def run_fused(packed, g, x, F, K, workspace=None, kind="gemv"):
    m = q4()
    M = x.shape[0]
    h = torch.full((M, F), -1, dtype=torch.int16, device=DEV)     # bf16 NaN pattern 0xFFFF
    fn = m.q4proj_gemv_silu_mul if kind == "gemv" else m.q4proj_gemm_silu_mul
    fn(packed[0], packed[1], g, to_dev_x(x), h, M, F, K, workspace=workspace)
    torch.cuda.synchronize()
    return h.cpu().numpy().view(np.uint16)


def assert_silu_parity(mat, x, F, h, cols=None):
    href, bound = oracle.silu_mul_cols(mat.codes, mat.scales, mat.g, x, F, cols=cols)
    hg = h if cols is None else h[:, cols]
    bad, worst = oracle.check_bf16(href, bound, hg)
    assert bad == 0, f"{bad} outputs outside the allowance (worst ratio {worst:.3g})"
    return worst


SMALL = [(M, F, K) for M in (1, 2, 3, 5, 7, 16) for F in (8, 40, 272) for K in (16, 208, 1040)]


@pytest.mark.parametrize("M,F,K", SMALL)
def test_small_shapes(M, F, K):
    mat = fused_matrix(40 + M, F, K)
    x = synth.x_bf16(40, M, M, K)
    note(f"gemv_silu_mul M={M} F={F} K={K}")
    h = run_fused(pack(mat.codes, mat.scales, 2 * F, K), mat.g, x, F, K)
    assert_silu_parity(mat, x, F, h)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_every_m(M):
    """Every M from 1 to 16: F = 2176 (272 row tiles, split between waves and
    workgroups) at K = 640, and F = 152 with two K ranges."""
    for j, (F, K) in enumerate([(2176, 640), (152, 128 * (512 // M + 4))]):
        mat = fused_matrix(70 + M + 20 * j, F, K)
        x = synth.x_bf16(70 + j, M, M, K)
        note(f"gemv_silu_mul M={M} F={F} K={K}")
        h = run_fused(pack(mat.codes, mat.scales, 2 * F, K), mat.g, x, F, K)
        assert_silu_parity(mat, x, F, h)


@pytest.mark.parametrize("M", [1, 130, 255])
def test_gemm_writes_no_row_past_m(M):
    """h is the first M rows of a larger buffer filled with a sentinel; the
    fused GEMM must leave every row past M untouched."""
    F, K = 136, 512
    mat = fused_matrix(95 + M, F, K)
    x = synth.x_bf16(95, M, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    big = torch.full((M + 256, F), 0x1234, dtype=torch.int16, device=DEV)
    note(f"gemm_silu_mul guard rows M={M} F={F} K={K}")
    q4().q4proj_gemm_silu_mul(packed[0], packed[1], mat.g, to_dev_x(x), big[:M], M, F, K)
    torch.cuda.synchronize()
    assert bool((big[M:].cpu() == 0x1234).all()), "rows past M were written"
    assert_silu_parity(mat, x, F, big[:M].cpu().numpy().view(np.uint16))


# Many row tiles per wave at short K (tiles complete inside one wave), and one
# shape with two K ranges.
WHOLE = [(1, 32768, 128), (3, 49152, 128), (4, 16384, 256), (16, 8192, 384), (2, 24592, 256),
         (13, 4096, 5120)]


@pytest.mark.parametrize("M,F,K", WHOLE)
def test_whole_tile_pairs(M, F, K):
    mat = fused_matrix(50, F, K)
    x = synth.x_bf16(50, M, M, K)
    note(f"gemv_silu_mul M={M} F={F} K={K}")
    h = run_fused(pack(mat.codes, mat.scales, 2 * F, K), mat.g, x, F, K)
    assert_silu_parity(mat, x, F, h)


def sample_cols(F, n, seed):
    rng = np.random.default_rng(seed)
    edge = np.array([0, 1, 7, 8, 9, F // 2, F - 9, F - 8, F - 1])
    return np.unique(np.concatenate([edge, rng.choice(F, n, replace=False)]))


@pytest.mark.parametrize("M", [1, 7, 16])
def test_decode_and_verify_full_size(M):
    (c,) = synth.workload_cases("mlp")
    mat, F, K = c.matrix, c.N // 2, c.K
    x = c.x if M == 1 else synth.x_bf16(5, 10 + M, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    ws = torch.zeros(q4().q4proj_silu_mul_workspace_bytes(M, F, K), dtype=torch.uint8, device=DEV)
    note(f"gemv_silu_mul M={M} F={F} K={K}")
    h1 = run_fused(packed, mat.g, x, F, K, workspace=ws)
    h2 = run_fused(packed, mat.g, x, F, K, workspace=ws)
    assert np.array_equal(h1, h2)
    assert int(torch.count_nonzero(ws)) == 0
    cols = sample_cols(F, 1024 if M == 1 else 256, M)
    worst = assert_silu_parity(mat, x, F, h1, cols)
    print(f"fused gate/up M={M}: worst |h-h_ref|/allowance = {worst:.3g}")


def bf16_round(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, nearest even (via fp32: exact for these magnitudes
    except on double-rounding ties, which the comparison below tolerates)."""
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


@pytest.mark.parametrize("M,F,K", [(1, 17408, 5120), (7, 4096, 1040), (16, 2048, 5120)])
def test_matches_unfused_gemv(M, F, K):
    mat = fused_matrix(60, F, K)
    x = synth.x_bf16(60, M, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    note(f"gemv_silu_mul vs gemv M={M} F={F} K={K}")
    h = run_fused(packed, mat.g, x, F, K)
    y = torch.empty((M, 2 * F), dtype=torch.float32, device=DEV)
    q4().q4proj_gemv(packed[0], packed[1], mat.g, to_dev_x(x), y, M, 2 * F, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    grow, urow = oracle.gate_up_rows(F)
    want = bf16_round(oracle.silu_mul(y[:, grow], y[:, urow]))
    # same fp32 gate/up sums; the epilogue's fp32 silu may move a result by
    # one bf16 step only where fp64 lies next to a rounding boundary
    diff = np.abs(h.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff == 0) > 0.995


def test_nan_scale_poisons_its_pair():
    F, K, M = 64, 256, 3
    mat = fused_matrix(70, F, K)
    scales = mat.scales.copy()
    scales[32 + 5, 3] = 0x7F              # fused row 37 = gate row of output f = 21
    scales[16 + 8 + 1, 0] = 0xFF          # fused row 25 = up row of output f = 9
    x = synth.x_bf16(70, M, M, K)
    note("gemv_silu_mul NaN scales")
    h = run_fused(pack(mat.codes, scales, 2 * F, K), mat.g, x, F, K)
    nan = (h & 0x7FFF) > 0x7F80
    assert nan[:, [9, 21]].all() and nan.sum() == 2 * M
    bad, _ = oracle.check_bf16(*oracle.silu_mul_cols(mat.codes, scales, mat.g, x, F), h)
    assert bad == 0


def test_rejects_what_it_does_not_serve():
    m = q4()
    KBIG = 288 * 128
    # one buffer stands in for both packed weights: as large as the packed
    # codes of the largest shape below, so no output range overlaps it
    w = torch.zeros(q4().q4proj_packed_codes_bytes(32, KBIG), dtype=torch.uint8, device=DEV)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    x = torch.zeros(16 * KBIG, dtype=torch.int16, device=DEV)
    h = torch.zeros(16 * 32, dtype=torch.int16, device=DEV)
    lib = m.library()

    def call(M, F, K):
        return lib.q4proj_gemv_silu_mul(w.data_ptr(), w.data_ptr(), 1.0, x.data_ptr(), h.data_ptr(),
                                        M, F, K, ws.data_ptr(), ws.numel(), None)

    # F % 8 != 0, M > 16, K past the eight-range limit at M = 16 (a range of
    # 36 k-tiles of 16 activation rows needs 147456 bytes of LDS, more than
    # the 147392 left beside the partial sums): rejected on the host, nothing
    # launched
    assert call(1, 12, 128) == m.EINVAL
    assert call(17, 16, 128) == m.EUNSUPPORTED
    assert call(16, 16, KBIG) == m.EUNSUPPORTED
    # the largest K served at M = 16: 35 k-tiles per range (143360 bytes);
    # all-zero weights give h = 0
    h.fill_(1)
    assert call(16, 16, 280 * 128) == m.OK
    torch.cuda.synchronize()
    assert int(h[:16 * 16].count_nonzero()) == 0


# ---- the matrix-core path (any M) ------------------------------------------

GEMM_SMALL = [(M, F, K) for M in (1, 33, 200) for F in (8, 40, 272) for K in (16, 208, 1040)]


@pytest.mark.parametrize("M,F,K", GEMM_SMALL)
def test_gemm_small_shapes(M, F, K):
    mat = fused_matrix(80 + M, F, K)
    x = synth.x_bf16(80, M, M, K)
    note(f"gemm_silu_mul M={M} F={F} K={K}")
    h = run_fused(pack(mat.codes, mat.scales, 2 * F, K), mat.g, x, F, K, kind="gemm")
    assert_silu_parity(mat, x, F, h)


# M = 512 with 3, 6, 9, 16 and 17 tiles per workgroup (every split of the
# tiles between the four wave pairs), on sampled outputs of every row
GEMM_TILINGS = [(1096, 256), (2816, 256), (4352, 128), (8192, 128), (17408, 5120)]


@pytest.mark.parametrize("F,K", GEMM_TILINGS)
def test_gemm_prefill_tilings(F, K):
    M = 512
    if F == 17408:
        (c,) = synth.workload_cases("pre", only=["gate_up"])
        x = c.x
        mat = synth.workload_cases("mlp")[0].matrix
    else:
        mat = fused_matrix(90, F, K)
        x = synth.x_bf16(90, 1, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    note(f"gemm_silu_mul M={M} F={F} K={K}")
    h1 = run_fused(packed, mat.g, x, F, K, kind="gemm")
    h2 = run_fused(packed, mat.g, x, F, K, kind="gemm")
    assert np.array_equal(h1, h2)
    cols = sample_cols(F, 256, F)
    worst = assert_silu_parity(mat, x, F, h1, cols)
    print(f"fused gate/up gemm F={F} K={K}: worst |h-h_ref|/allowance = {worst:.3g}")


@pytest.mark.parametrize("M,F,K", [(512, 4352, 1040), (77, 2048, 5120)])
def test_gemm_matches_unfused(M, F, K):
    mat = fused_matrix(100, F, K)
    x = synth.x_bf16(100, M, M, K)
    packed = pack(mat.codes, mat.scales, 2 * F, K)
    note(f"gemm_silu_mul vs gemm M={M} F={F} K={K}")
    h = run_fused(packed, mat.g, x, F, K, kind="gemm")
    y = torch.empty((M, 2 * F), dtype=torch.float32, device=DEV)
    q4().q4proj_gemm(packed[0], packed[1], mat.g, to_dev_x(x), y, M, 2 * F, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    grow, urow = oracle.gate_up_rows(F)
    want = bf16_round(oracle.silu_mul(y[:, grow], y[:, urow]))
    diff = np.abs(h.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff == 0) > 0.995


def test_gemm_nan_scale_poisons_its_pair():
    F, K, M = 64, 256, 40
    mat = fused_matrix(70, F, K)
    scales = mat.scales.copy()
    scales[32 + 5, 3] = 0x7F              # fused row 37 = gate row of output f = 21
    scales[16 + 8 + 1, 0] = 0xFF          # fused row 25 = up row of output f = 9
    x = synth.x_bf16(71, M, M, K)
    note("gemm_silu_mul NaN scales")
    h = run_fused(pack(mat.codes, scales, 2 * F, K), mat.g, x, F, K, kind="gemm")
    nan = (h & 0x7FFF) > 0x7F80
    assert nan[:, [9, 21]].all() and nan.sum() == 2 * M
    bad, _ = oracle.check_bf16(*oracle.silu_mul_cols(mat.codes, scales, mat.g, x, F), h)
    assert bad == 0

