"""Prepared calls (prepare_*): the eager call's checks run once and the
returned launcher calls the C entry point with converted arguments.  Each
launcher's results must equal the eager call's bit for bit, on repeated
launches; errors the library reports at call time are raised; and a
prepared call keeps its tensors alive."""
import gc

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K):
    mat = synth.nvfp4_normal_matrix(seed, 1, N, K, threads=4)
    pc, ps = pack(mat.codes, mat.scales, N, K)
    x = to_dev_x(synth.x_bf16(seed, 2, M, K, threads=1))
    return mat, pc, ps, x


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("kind,M,N,K", [("gemv", 1, 17408, 5120), ("gemv", 7, 5120, 17408),
                                        ("gemv_noalloc", 3, 4096, 2560),
                                        ("gemm", 300, 1040, 2064)])
def test_prepared_projection_matches_eager(kind, M, N, K):
    m = q4()
    mat, pc, ps, x = _inputs(80 + M, M, N, K)
    y_eager = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    y_prep = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    note(f"prepared {kind} M={M} N={N} K={K}")
    getattr(m, "q4proj_" + kind)(pc, ps, mat.g, x, y_eager, M, N, K)
    launch = getattr(m, "prepare_" + kind)(pc, ps, mat.g, x, y_prep, M, N, K)
    for _ in range(5):
        y_prep.fill_(float("nan"))
        launch()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_prep), _bits(y_eager))


@pytest.mark.parametrize("kind,M", [("gemv_silu_mul", 2), ("gemm_silu_mul", 64)])
def test_prepared_silu_matches_eager(kind, M):
    m = q4()
    F, K = 1024, 2560
    mat, pc, ps, x = _inputs(90 + M, M, 2 * F, K)
    h_eager = torch.zeros((M, F), dtype=torch.int16, device=DEV)
    h_prep = torch.full((M, F), -1, dtype=torch.int16, device=DEV)
    note(f"prepared {kind} M={M} F={F} K={K}")
    getattr(m, "q4proj_" + kind)(pc, ps, mat.g, x, h_eager, M, F, K)
    launch = getattr(m, "prepare_" + kind)(pc, ps, mat.g, x, h_prep, M, F, K)
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    assert torch.equal(h_prep, h_eager)


def test_prepared_argmax_matches_eager():
    m = q4()
    M, N, K = 4, 65536, 2560
    mat, pc, ps, x = _inputs(95, M, N, K)
    val_e = torch.empty(M, dtype=torch.float32, device=DEV)
    idx_e = torch.empty(M, dtype=torch.int64, device=DEV)
    val_p = torch.empty(M, dtype=torch.float32, device=DEV)
    idx_p = torch.empty(M, dtype=torch.int64, device=DEV)
    note(f"prepared gemv_argmax M={M} N={N} K={K}")
    m.q4proj_gemv_argmax(pc, ps, mat.g, x, None, val_e, idx_e, M, N, K)
    launch = m.prepare_gemv_argmax(pc, ps, mat.g, x, None, val_p, idx_p, M, N, K)
    for _ in range(4):
        launch()
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_e) and torch.equal(val_p.view(torch.int32), val_e.view(torch.int32))


def test_prepared_call_raises_library_errors():
    m = q4()
    M, N, K = 17, 256, 512                      # the GEMV serves M <= 16
    mat, pc, ps, x = _inputs(96, M, N, K)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    launch = m.prepare_gemv(pc, ps, mat.g, x, y, M, N, K, workspace=ws)
    with pytest.raises(m.Q4ProjError) as e:
        launch()
    assert e.value.status == m.EUNSUPPORTED


def test_prepared_call_keeps_its_tensors():
    m = q4()
    M, N, K = 1, 2048, 1024
    mat, pc, ps, x = _inputs(97, M, N, K)
    y_ref = torch.empty((M, N), dtype=torch.float32, device=DEV)
    m.q4proj_gemv(pc, ps, mat.g, x, y_ref, M, N, K)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y_addr = y.data_ptr()
    launch = m.prepare_gemv(pc, ps, mat.g, x, y, M, N, K)
    del pc, ps, x                                # only the launcher holds them now
    gc.collect()
    scratch = [torch.full((1 << 20,), 7, dtype=torch.uint8, device=DEV) for _ in range(8)]
    launch()
    torch.cuda.synchronize()
    assert y.data_ptr() == y_addr
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    del scratch
