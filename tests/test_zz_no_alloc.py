"""q4proj_gemv_noalloc (the GEMV whose exchange words live in the library's
per-GPU scratch array) against q4proj_gemv with a caller workspace, through
the C ABI: bit for bit, on two calls in a row, the second on a smaller shape
than the first (the array keeps the first call's contents: every completed
call must leave it zero-filled), then on the first shape again; and the
refusal of a shape beyond the array's 8 MiB."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, assert_parity, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K):
    mat = synth.nvfp4_normal_matrix(seed, 1, N, K, threads=8)
    x = synth.x_bf16(seed, 2, M, K, threads=1)
    pc, ps = pack(mat.codes, mat.scales, N, K)
    return mat, x, pc, ps, to_dev_x(x)


def _noalloc(lib, pc, ps, g, xd, y, M, N, K):
    st = torch.cuda.current_stream().cuda_stream
    return lib.q4proj_gemv_noalloc(pc.data_ptr(), ps.data_ptr(), ctypes.c_float(g), xd.data_ptr(),
                                   y.data_ptr(), M, N, K, ctypes.c_void_p(st))


def test_noalloc_matches_gemv_on_consecutive_calls():
    m = q4()
    lib = m.library()
    # larger first (two K ranges: join words beyond the boundary words), then
    # a smaller shape, then the first again
    shapes = [(7, 5120, 17408), (1, 2560, 9216), (7, 5120, 17408), (3, 300, 1040)]
    cache = {}
    for i, (M, N, K) in enumerate(shapes):
        if (M, N, K) not in cache:
            cache[(M, N, K)] = _inputs(70 + len(cache), M, N, K)
        mat, x, pc, ps, xd = cache[(M, N, K)]
        y0 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        note(f"gemv_noalloc call {i}: M={M} N={N} K={K}")
        assert _noalloc(lib, pc, ps, mat.g, xd, y1, M, N, K) == m.OK
        ws = torch.zeros(m.q4proj_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
        m.q4proj_gemv(pc, ps, mat.g, xd, y0, M, N, K, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"call {i}: noalloc differs from gemv"
        if i == 0:
            assert_parity(mat.codes, mat.scales, mat.g, x, y1.cpu().numpy())


def test_noalloc_refuses_beyond_its_array():
    m = q4()
    lib = m.library()
    M, N, K = 16, 248320, 5120
    assert m.q4proj_workspace_bytes(M, N, K) > 8 << 20
    pc = torch.empty(m.q4proj_packed_codes_bytes(N, K), dtype=torch.uint8, device=DEV)
    ps = torch.empty(m.q4proj_packed_scales_bytes(N, K), dtype=torch.uint8, device=DEV)
    xd = torch.zeros((M, K), dtype=torch.int16, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    assert _noalloc(lib, pc, ps, 1.0, xd, y, M, N, K) == m.EWORKSPACE
