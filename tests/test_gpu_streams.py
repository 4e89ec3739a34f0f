"""Calls on streams other than the current one, and on two streams at once,
with the binding's default workspaces (one per device and stream, allocated
and zero-filled on that stream).

* gemv on two streams concurrently, several calls queued on each before any
  synchronisation, every result against the oracle;
* gemv, gemv_silu_mul, gemv_argmax and quantize on a non-default stream with
  no explicit workspace, against the oracle;
* the default workspaces of two streams are distinct buffers.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_parity, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def _case(seed, M, N, K):
    mat = synth.nvfp4_normal_matrix(seed, 1, N, K, threads=4)
    x = synth.x_bf16(seed, 2, M, K, threads=1)
    return mat, x


def test_default_workspaces_are_per_stream():
    m = q4()
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    wa = m.default_workspace(0, 4096, a)
    wb = m.default_workspace(0, 4096, b)
    assert wa.data_ptr() != wb.data_ptr()
    assert m.default_workspace(0, 4096, a).data_ptr() == wa.data_ptr()
    torch.cuda.synchronize()
    assert int(wa.count_nonzero()) == 0 and int(wb.count_nonzero()) == 0


@pytest.mark.parametrize("M,N,K", [(1, 17408, 5120), (7, 5120, 17408)])
def test_gemv_two_streams_concurrently(M, N, K):
    m = q4()
    cases = [_case(40 + i, M, N, K) for i in range(2)]
    dev_in = []
    for mat, x in cases:
        pc, ps = pack(mat.codes, mat.scales, N, K)
        dev_in.append((pc, ps, mat.g, to_dev_x(x)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    reps = 6
    ys = [[torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV) for _ in range(reps)]
          for _ in streams]
    torch.cuda.synchronize()                   # inputs and outputs ready before the side streams
    note(f"gemv on two streams, {reps} calls each, M={M} N={N} K={K}")
    # queue the calls alternately so that the two streams' kernels overlap
    for r in range(reps):
        for i, st in enumerate(streams):
            pc, ps, g, xd = dev_in[i]
            with torch.cuda.stream(st):
                m.q4proj_gemv(pc, ps, g, xd, ys[i][r], M, N, K, stream=st)
    torch.cuda.synchronize()
    for i, (mat, x) in enumerate(cases):
        first = ys[i][0].cpu().numpy()
        assert_parity(mat.codes, mat.scales, mat.g, x, first)
        for r in range(1, reps):
            assert torch.equal(ys[i][r], ys[i][0]), f"stream {i} call {r} differs"
    for st in streams:
        ws = m.default_workspace(0, m.q4proj_workspace_bytes(M, N, K), st)
        assert int(ws.count_nonzero()) == 0, "workspace not left zero-filled"


def test_entry_points_on_a_side_stream():
    m = q4()
    st = torch.cuda.Stream()
    # plain projection
    M, N, K = 3, 4096, 2560
    mat, x = _case(50, M, N, K)
    pc, ps = pack(mat.codes, mat.scales, N, K)
    xd = to_dev_x(x)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    val = torch.empty(M, dtype=torch.float32, device=DEV)
    idx = torch.empty(M, dtype=torch.int64, device=DEV)
    torch.cuda.synchronize()
    note("gemv on a side stream")
    m.q4proj_gemv(pc, ps, mat.g, xd, y, M, N, K, stream=st)
    st.synchronize()
    assert_parity(mat.codes, mat.scales, mat.g, x, y.cpu().numpy())
    # greedy argmax
    note("gemv_argmax on a side stream")
    m.q4proj_gemv_argmax(pc, ps, mat.g, xd, None, val, idx, M, N, K, stream=st)
    st.synchronize()
    yr, S = oracle.proj(mat.codes, mat.scales, mat.g, x)
    assert oracle.argmax_check(yr, S, idx.cpu().numpy(), val.cpu().numpy()) == 0
    # fused gate/up + silu * up
    F, Kf, Mf = 256, 1024, 2
    fm = synth.nvfp4_normal_matrix(51, 1, 2 * F, Kf, threads=4)
    xf = synth.x_bf16(51, 2, Mf, Kf, threads=1)
    fpc, fps = pack(fm.codes, fm.scales, 2 * F, Kf)
    xfd = to_dev_x(xf)
    h = torch.empty((Mf, F), dtype=torch.int16, device=DEV)
    torch.cuda.synchronize()
    note("gemv_silu_mul on a side stream")
    m.q4proj_gemv_silu_mul(fpc, fps, fm.g, xfd, h, Mf, F, Kf, stream=st)
    st.synchronize()
    h_ref, bound = oracle.silu_mul_cols(fm.codes, fm.scales, fm.g, xf, F)
    bad, _ = oracle.check_bf16(h_ref, bound, h.cpu().numpy().view(np.uint16))
    assert bad == 0
    # quantizer (temporary workspace allocated on the side stream)
    Nq, Kq = 48, 640
    wb = synth.normal_bf16(52, 1, Nq * Kq, std=0.02)
    wd = torch.from_numpy(wb.view(np.int16)).to(DEV)
    torch.cuda.synchronize()
    note("quantize on a side stream")
    codes, scales, g = m.quantize_weight(wd, Nq, Kq, stream=st)
    st.synchronize()
    rc, rs, rg = oracle.quantize(wb, Nq, Kq)
    assert float(g.item()) == rg
    assert np.array_equal(codes.cpu().numpy().reshape(Nq, -1), rc)
    assert np.array_equal(scales.cpu().numpy().reshape(Nq, -1), rs)
