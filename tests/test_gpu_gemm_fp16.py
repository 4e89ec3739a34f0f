"""The GEMMs' fp16 operand path (with a staging workspace) against the bf16
path (without one) and the CPU oracle.

With a workspace, q4proj_gemm / q4proj_gemm_silu_mul first copy each
activation row to fp16 scaled by 2^-c, c = (largest exponent of the row's
nonzero values) - 15, with the output multiplier g * 2^c per row, or NaN for
a row fp16 cannot hold exactly (nonzero magnitudes spanning more than 29
binades, an infinity or NaN, or g * 2^c outside the normal floats); a
128-row block with such a row runs on bf16 operands.  Both paths multiply exact products and sum them
in the same order, so their outputs must agree bit for bit.

* the staging step (the workspace after a call) against its definition,
  written out here in numpy, on rows at and past the 29-binade boundary,
  bf16 subnormals, infinities, NaNs, zeros and very large values;
* fp16 and bf16 paths bitwise equal on those rows (NaN positions equal), on
  ragged shapes and on the full M = 512 prefill shapes, plain and fused;
* every finite row within the oracle's tolerance;
* rows longer than the 8192 values the staging kernel keeps in registers,
  with their extremes, an infinity and a NaN past that point;
* one workspace reused by calls of different sizes, no contents required.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_parity, bits, gemm_workspace, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def r256(n):
    return -(-n // 256) * 256


def staging_model(x: np.ndarray, g: float):
    """(fp16 copy, row multipliers) the staging step must write: the
    definition above in float32/float16 numpy arithmetic (the copy matters
    only for rows whose multiplier is not NaN)."""
    f = (x.astype(np.uint32) << 16).view(np.float32)
    M = x.shape[0]
    xh = np.zeros(x.shape, dtype=np.float16)
    rowmul = np.zeros(M, dtype=np.float32)
    for m in range(M):
        row = f[m]
        live = row != 0
        if not np.isfinite(row).all():
            rowmul[m] = np.float32(np.nan)
            continue
        if live.any():
            ex = np.frexp(row[live])[1].astype(np.int64) - 1          # floor(log2 |v|)
            hi, lo = int(ex.max()), int(ex.min())
            c = hi - 15
            exact = lo - c >= -14
        else:
            c, exact = 0, True
        with np.errstate(over="ignore", under="ignore"):
            gm = np.ldexp(np.float32(g), c).astype(np.float32)
            xh[m] = np.ldexp(row, -c).astype(np.float16)
        mul_ok = g == 0 or (np.finfo(np.float32).tiny <= abs(gm) <= np.finfo(np.float32).max)
        rowmul[m] = gm if (exact and mul_ok) else np.float32(np.nan)
    return xh, rowmul


def bf16(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def special_rows(M, K, seed):
    """N(0,1) activations with special rows: rows 0..127 all convert exactly
    (fp16 path), rows 128..255 include ones that do not (bf16 fallback for
    that block), rows 256.. are plain."""
    x = synth.x_bf16(seed, 9, M, K)
    x[6] = 0                                     # 29 binades: exact at the boundary
    x[6, 0], x[6, 1] = bf16(1.5 * 2.0 ** 10), bf16(2.0 ** -19)
    x[7, 40] = bf16(2.0 ** -25)                  # a subnormal in fp16 without the scaling
    x[11] = 0                                    # all zero
    x[150, 17] = 0x7F80                          # +Inf
    x[151, 3] = 0x7FC0                           # NaN
    x[12] = ((x[12].astype(np.uint32) + (100 << 7)) & 0xFFFF).astype(np.uint16)  # x * 2^100
    x[133] = 0                                   # 30 binades: inexact
    x[133, 0], x[133, 1] = bf16(2.0 ** 20), bf16(2.0 ** -10)
    x[135] = 0
    x[135, 5], x[135, 900] = bf16(2.0 ** 10), bf16(2.0 ** -20)
    rng = np.random.default_rng(seed)
    x[140] = rng.integers(1, 128, K).astype(np.uint16) | (rng.integers(0, 2, K).astype(np.uint16) << 15)
    return x


def run_gemm(packed, g, x, N, K, workspace):
    M = x.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q4().q4proj_gemm(packed[0], packed[1], g, to_dev_x(x), y, M, N, K, workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def run_silu(packed, g, x, F, K, workspace):
    M = x.shape[0]
    h = torch.full((M, F), -1, dtype=torch.int16, device=DEV)
    q4().q4proj_gemm_silu_mul(packed[0], packed[1], g, to_dev_x(x), h, M, F, K,
                              workspace=workspace)
    torch.cuda.synchronize()
    return h.cpu().numpy().view(np.uint16)


def same_bits_nan_aware(a: np.ndarray, b: np.ndarray) -> bool:
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(bits(a)[~na], bits(b)[~nb])


def test_staging_and_paths_on_special_rows():
    m = q4()
    M, N, K = 300, 272, 1040
    w = synth.nvfp4_normal_matrix(71, 1, N, K)
    x = special_rows(M, K, 71)
    packed = pack(w.codes, w.scales, N, K)
    need = m.q4proj_gemm_workspace_bytes(M, N, K)
    assert need == r256(2 * M * K) + r256(4 * M)
    ws = torch.full((need,), 0xAA, dtype=torch.uint8, device=DEV)   # no contents required
    note(f"gemm fp16 staging M={M} N={N} K={K}")
    y16 = run_gemm(packed, w.g, x, N, K, ws)
    wsh = ws.cpu().numpy()
    xh = wsh[:2 * M * K].view(np.float16).reshape(M, K)
    rowmul = wsh[r256(2 * M * K):r256(2 * M * K) + 4 * M].view(np.float32)
    xh_ref, rowmul_ref = staging_model(x, w.g)
    nan_rows = np.flatnonzero(np.isnan(rowmul_ref))
    assert list(nan_rows) == [133, 135, 140, 150, 151], nan_rows
    assert np.array_equal(np.isnan(rowmul), np.isnan(rowmul_ref))
    ok = ~np.isnan(rowmul_ref)
    assert np.array_equal(rowmul[ok].view(np.uint32), rowmul_ref[ok].view(np.uint32))
    for r in np.flatnonzero(ok):
        assert same_bits_nan_aware(xh[r].astype(np.float32), xh_ref[r].astype(np.float32)), r
        # exact: the fp16 copy times 2^c gives back the bf16 values
        f = (x[r].astype(np.uint32) << 16).view(np.float32)
        back = xh[r].astype(np.float64) * (float(rowmul_ref[r]) / w.g if w.g else 1.0)
        fin = np.isfinite(f)
        assert np.array_equal(back[fin], f[fin].astype(np.float64)), r

    note("gemm bf16 path on the same rows")
    y32 = run_gemm(packed, w.g, x, N, K, False)
    assert same_bits_nan_aware(y16, y32)
    # rows of finite activations against the oracle (row 140, bf16 subnormals
    # only, runs on bf16 operands like the path without a workspace, which
    # the paths' equality above covers)
    finite_rows = np.flatnonzero(np.isfinite((x.astype(np.uint32) << 16).view(np.float32)).all(1))
    finite_rows = finite_rows[finite_rows != 140]
    assert_parity(w.codes, w.scales, w.g, x, y16, xrows=finite_rows)
    assert np.isinf(y16[150]).any() or np.isnan(y16[150]).any()
    assert np.isnan(y16[151]).all()
    assert (y16[11] == 0).all()

    F = N // 2
    note(f"gemm_silu_mul fp16 vs bf16 M={M} F={F} K={K}")
    h16 = run_silu(packed, w.g, x, F, K, ws)
    h32 = run_silu(packed, w.g, x, F, K, False)
    nan16, nan32 = (h16 & 0x7FFF) > 0x7F80, (h32 & 0x7FFF) > 0x7F80
    assert np.array_equal(nan16, nan32) and np.array_equal(h16[~nan16], h32[~nan32])


def test_staging_long_rows():
    """Rows longer than the 8192 values the staging kernel holds in
    registers: the chunks past them are scanned and converted on a second
    read, so the row's extremes are placed there."""
    m = q4()
    M, N, K = 136, 64, 12304
    w = synth.nvfp4_normal_matrix(91, 1, N, K)
    x = synth.x_bf16(91, 9, M, K)
    x[1, 12000] = bf16(2.0 ** 12)                # the row's largest value, past 8192
    # row 2: magnitudes capped at 0.5 (largest exponent -1) and one 2^-30
    # past 8192: 29 binades, exact at the boundary
    x[2] = np.where(np.abs((x[2].astype(np.uint32) << 16).view(np.float32)) > 0.5,
                    bf16(0.25), x[2]).astype(np.uint16)
    x[2, 10] = bf16(0.5)
    x[2, 9000] = bf16(2.0 ** -30)
    x[130] = 0                                   # 30 binades, the small end past 8192
    x[130, 5], x[130, 10000] = bf16(2.0 ** 20), bf16(2.0 ** -10)
    x[131, 11000] = 0x7F80                       # +Inf past 8192
    x[132, K - 1] = 0xFFC0                       # NaN in the last chunk
    packed = pack(w.codes, w.scales, N, K)
    need = m.q4proj_gemm_workspace_bytes(M, N, K)
    ws = torch.full((need,), 0x55, dtype=torch.uint8, device=DEV)
    note(f"gemm fp16 staging, long rows M={M} N={N} K={K}")
    y16 = run_gemm(packed, w.g, x, N, K, ws)
    wsh = ws.cpu().numpy()
    xh = wsh[:2 * M * K].view(np.float16).reshape(M, K)
    rowmul = wsh[r256(2 * M * K):r256(2 * M * K) + 4 * M].view(np.float32)
    xh_ref, rowmul_ref = staging_model(x, w.g)
    assert list(np.flatnonzero(np.isnan(rowmul_ref))) == [130, 131, 132]
    assert np.array_equal(np.isnan(rowmul), np.isnan(rowmul_ref))
    ok = ~np.isnan(rowmul_ref)
    assert np.array_equal(rowmul[ok].view(np.uint32), rowmul_ref[ok].view(np.uint32))
    for r in np.flatnonzero(ok):
        assert np.array_equal(xh[r].view(np.uint16), xh_ref[r].view(np.uint16)), r
    note("gemm bf16 path on the same rows")
    y32 = run_gemm(packed, w.g, x, N, K, False)
    assert same_bits_nan_aware(y16, y32)
    assert_parity(w.codes, w.scales, w.g, x, y16, xrows=np.arange(128))


@pytest.mark.parametrize("M,N,K", [(129, 300, 1040), (513, 100, 272), (1, 17, 5136), (3, 40, 16),
                                   (200, 4112, 128), (64, 2049, 400), (300, 48, 2000)])
def test_fp16_and_bf16_paths_agree_bitwise(M, N, K):
    w = synth.nvfp4_normal_matrix(80 + M, 3, N, K)
    x = synth.x_bf16(80 + M, 4, M, K)
    packed = pack(w.codes, w.scales, N, K)
    note(f"gemm fp16/bf16 M={M} N={N} K={K}")
    ws = gemm_workspace(M, N, K)
    y16 = run_gemm(packed, w.g, x, N, K, ws)
    y32 = run_gemm(packed, w.g, x, N, K, False)
    assert np.array_equal(bits(y16), bits(y32))
    assert_parity(w.codes, w.scales, w.g, x, y16)
    if N % 16 == 0:
        F = N // 2
        note(f"gemm_silu_mul fp16/bf16 M={M} F={F} K={K}")
        assert np.array_equal(run_silu(packed, w.g, x, F, K, ws),
                              run_silu(packed, w.g, x, F, K, False))


@pytest.mark.parametrize("N,silu", [(14336, False), (17408, False), (34816, True)])
def test_full_size_prefill_paths_agree(N, silu):
    """The M = 512 prefill chunk on the qkv and gate/up weights and the fused
    gate/up + SiLU: the fp16 path bit for bit equal to the bf16 path over
    every output, and sampled outputs against the oracle."""
    m = q4()
    M, K = 512, 5120
    w = synth.nvfp4_normal_matrix(90, 1, N, K)
    x = synth.x_bf16(90, 2, M, K)
    packed = pack(w.codes, w.scales, N, K)
    xd = to_dev_x(x)
    wsp = gemm_workspace(M, N, K)
    if silu:
        F = N // 2
        outs = [torch.full((M, F), -1, dtype=torch.int16, device=DEV) for _ in range(2)]
        for o, ws in zip(outs, (wsp, False)):
            note(f"gemm_silu_mul M={M} F={F} K={K} staged={ws is not False}")
            m.q4proj_gemm_silu_mul(packed[0], packed[1], w.g, xd, o, M, F, K, workspace=ws)
    else:
        outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
        for o, ws in zip(outs, (wsp, False)):
            note(f"gemm M={M} N={N} K={K} staged={ws is not False}")
            m.q4proj_gemm(packed[0], packed[1], w.g, xd, o, M, N, K, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    rows = np.array([0, 1, 127, 128, 300, 511])
    if silu:
        cols = np.array([0, 7, 8, 4095, 8703, 17407])
        href, bound = oracle.silu_mul_cols(w.codes, w.scales, w.g, x[rows], N // 2, cols=cols)
        hg = outs[0].cpu().numpy().view(np.uint16)[rows][:, cols]
        bad, _ = oracle.check_bf16(href, bound, hg)
        assert bad == 0
    else:
        cols = np.array([0, 15, 16, 5000, N - 17, N - 1])
        assert_parity(w.codes, w.scales, w.g, x, outs[0].cpu().numpy(), rows=cols, xrows=rows)


def test_workspace_reused_across_sizes():
    """One explicit workspace for a large call and then a smaller one (its
    contents are scratch): both match the bf16 path bit for bit."""
    m = q4()
    N, K = 272, 1040
    w = synth.nvfp4_normal_matrix(95, 1, N, K)
    packed = pack(w.codes, w.scales, N, K)
    ws = torch.empty(m.q4proj_gemm_workspace_bytes(400, N, K), dtype=torch.uint8, device=DEV)
    for M in (400, 130):
        x = synth.x_bf16(95, M, M, K)
        note(f"gemm shared workspace M={M}")
        y16 = run_gemm(packed, w.g, x, N, K, ws)
        y32 = run_gemm(packed, w.g, x, N, K, False)
        assert np.array_equal(bits(y16), bits(y32))
        assert_parity(w.codes, w.scales, w.g, x, y16)

