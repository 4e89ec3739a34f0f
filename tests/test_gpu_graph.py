"""The entry points inside a captured HIP graph.

The FlashRT "Qwen3.6 NVFP4 usage" page's constructor-argument table has the
runner pre-allocate every per-step buffer so that no call allocates and the
decode step can be captured as a graph.  Here one graph holds the decode GEMV
(M = 1), the verify GEMV (M = 7 with K = 17408: K ranges joined through the
workspace), the GEMM, the fused gate/up GEMV, the lm-head-style argmax
(no logits) and the quantizer, each with a caller-provided workspace.  The
graph is replayed several times; before each replay new activations and a new
bf16 weight are copied into its input buffers and the device synchronised
(eager work between replays), and after it every output must equal the eager
calls on the same inputs bit for bit (every kernel here is deterministic).
The decode GEMV's first replay is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu


def _weight(seed, N, K):
    mat = synth.nvfp4_normal_matrix(seed, 1, N, K, threads=1)
    return mat, pack(mat.codes, mat.scales, N, K)


def test_graph_replays_match_eager_bit_for_bit():
    m = q4()
    # (name, M, N, K) of the projections in the graph
    dec_mat, dec_w = _weight(31, 1040, 2048)
    ver_mat, ver_w = _weight(32, 640, 17408)
    pre_mat, pre_w = _weight(33, 272, 1024)
    F, Kf = 200, 512
    mlp_mat, mlp_w = _weight(34, 2 * F, Kf)
    lm_mat, lm_w = _weight(35, 5000, 256)
    Nq, Kq = 48, 640

    xs = {"dec": torch.zeros((1, 2048), dtype=torch.int16, device=DEV),
          "ver": torch.zeros((7, 17408), dtype=torch.int16, device=DEV),
          "pre": torch.zeros((40, 1024), dtype=torch.int16, device=DEV),
          "mlp": torch.zeros((1, Kf), dtype=torch.int16, device=DEV),
          "lm": torch.zeros((1, 256), dtype=torch.int16, device=DEV)}
    wq = torch.zeros(Nq * Kq, dtype=torch.int16, device=DEV)
    ws = {"dec": torch.zeros(m.q4proj_workspace_bytes(1, 1040, 2048), dtype=torch.uint8, device=DEV),
          "ver": torch.zeros(m.q4proj_workspace_bytes(7, 640, 17408), dtype=torch.uint8, device=DEV),
          "mlp": torch.zeros(m.q4proj_silu_mul_workspace_bytes(1, F, Kf), dtype=torch.uint8,
                             device=DEV),
          "lm": torch.zeros(m.q4proj_argmax_workspace_bytes(1, 5000, 256), dtype=torch.uint8,
                            device=DEV),
          "quant": torch.zeros(m.q4proj_quantize_workspace_bytes(Nq, Kq), dtype=torch.uint8,
                               device=DEV),
          # the GEMM's fp16 staging scratch (no contents required)
          "pre": torch.empty(m.q4proj_gemm_workspace_bytes(40, 272, 1024), dtype=torch.uint8,
                             device=DEV)}

    def outputs():
        return {"dec": torch.full((1, 1040), float("nan"), device=DEV),
                "ver": torch.full((7, 640), float("nan"), device=DEV),
                "pre": torch.full((40, 272), float("nan"), device=DEV),
                "mlp": torch.full((1, F), -1, dtype=torch.int16, device=DEV),
                "val": torch.full((1,), -1.0, device=DEV),
                "idx": torch.full((1,), -1, dtype=torch.int64, device=DEV),
                "qc": torch.full((Nq * Kq // 2,), 0xAA, dtype=torch.uint8, device=DEV),
                "qs": torch.full((Nq * Kq // 16,), 0xAA, dtype=torch.uint8, device=DEV),
                "qg": torch.full((1,), -1.0, device=DEV)}

    def step(o):
        m.q4proj_gemv(dec_w[0], dec_w[1], dec_mat.g, xs["dec"], o["dec"], 1, 1040, 2048,
                      workspace=ws["dec"])
        m.q4proj_gemv(ver_w[0], ver_w[1], ver_mat.g, xs["ver"], o["ver"], 7, 640, 17408,
                      workspace=ws["ver"])
        m.q4proj_gemm(pre_w[0], pre_w[1], pre_mat.g, xs["pre"], o["pre"], 40, 272, 1024,
                      workspace=ws["pre"])
        m.q4proj_gemv_silu_mul(mlp_w[0], mlp_w[1], mlp_mat.g, xs["mlp"], o["mlp"], 1, F, Kf,
                               workspace=ws["mlp"])
        m.q4proj_gemv_argmax(lm_w[0], lm_w[1], lm_mat.g, xs["lm"], None, o["val"], o["idx"],
                             1, 5000, 256, workspace=ws["lm"])
        m.q4proj_quantize(wq, Nq, Kq, o["qc"], o["qs"], o["qg"], workspace=ws["quant"])

    def load_inputs(rep):
        for j, (k, x) in enumerate(xs.items()):
            x.copy_(to_dev_x(synth.x_bf16(40 + rep, j, x.shape[0], x.shape[1], threads=1)))
        wq.copy_(torch.from_numpy(synth.normal_bf16(50 + rep, 1, Nq * Kq, std=0.02)
                                  .view(np.int16)).to(DEV))
        torch.cuda.synchronize()

    note("graph: eager warm-up")
    load_inputs(0)
    warm = outputs()
    step(warm)
    torch.cuda.synchronize()

    note("graph: capture")
    graph_out = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graph_out)
    torch.cuda.synchronize()

    for rep in range(1, 5):
        note(f"graph: replay {rep}")
        load_inputs(rep)
        for t in graph_out.values():
            t.fill_(0x55 if t.dtype == torch.uint8 else -3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = outputs()
        step(eager)
        torch.cuda.synchronize()
        for k in eager:
            a, b = graph_out[k], eager[k]
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager call"
        if rep == 1:
            x = xs["dec"].cpu().numpy().view(np.uint16)
            yr, S = oracle.proj(dec_mat.codes, dec_mat.scales, dec_mat.g, x)
            bad, _ = oracle.check(yr, S, graph_out["dec"].cpu().numpy())
            assert bad == 0
    # the workspaces are left zero-filled by every call, replays included
    for k, w in ws.items():
        if k not in ("quant", "pre"):
            assert int(torch.count_nonzero(w)) == 0, f"{k} workspace not left zero-filled"
