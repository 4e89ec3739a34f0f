"""Helpers for the GPU parity tests: move synthetic inputs to the device, run
the HIP entry points through the binding, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def note(msg: str):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def q4():
    import nvfp4_weight_only_q4proj_amd as mod
    return mod


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_dev_x(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).to(DEV)


def pack(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    m = q4()
    return m.pack_weight(to_dev_u8(codes).reshape(-1), to_dev_u8(scales).reshape(-1), N, K)


def project(kind: str, packed, g: float, x: np.ndarray, N: int, K: int) -> np.ndarray:
    m = q4()
    M = x.shape[0]
    xd = to_dev_x(x)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    if kind == "gemv":
        m.q4proj_gemv(packed[0], packed[1], g, xd, y, M, N, K)
    else:
        # "gemm": fp16 operands (an explicit staging workspace, whatever the
        # shape); "gemm_bf16": no workspace, bf16 operands
        ws = False if kind == "gemm_bf16" else gemm_workspace(M, N, K)
        m.q4proj_gemm(packed[0], packed[1], g, xd, y, M, N, K, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gemm_workspace(M: int, N: int, K: int) -> torch.Tensor:
    """A staging workspace for the GEMMs (fp16 operands), filled with a
    pattern: it needs no contents."""
    return torch.full((q4().q4proj_gemm_workspace_bytes(M, N, K),), 0xA5, dtype=torch.uint8,
                      device=DEV)


def run(kind: str, codes, scales, g, x) -> np.ndarray:
    N = codes.shape[0]
    K = codes.shape[1] * 2
    note(f"{kind} M={x.shape[0]} N={N} K={K}")
    return project(kind, pack(codes, scales, N, K), g, x, N, K)


def assert_parity(codes, scales, g, x, y, rows=None, xrows=None, diag=1e-5):
    """Every checked element within |y - y_ref| <= 2e-3 * S.  Also asserts the
    diagnostic max |y - y_ref| / S <= diag (a fp32 accumulation of exact
    products stays orders of magnitude below the gate; a decode slip does not).
    rows: weight rows (columns of y) to check; xrows: activation rows."""
    xs = x if xrows is None else x[xrows]
    yr, S = oracle.proj_rows(codes, scales, g, xs, rows)
    yg = y if xrows is None else y[xrows]
    if rows is not None:
        yg = yg[:, rows]
    bad, worst = oracle.check(yr, S, yg)
    assert bad == 0, f"{bad} elements outside tolerance (worst ratio {worst:.3g})"
    assert worst <= diag, f"max |y-y_ref|/S = {worst:.3g} above the {diag:g} diagnostic bound"
    return worst


def oracle_fp32(codes, scales, g, x, rows=None):
    y, _ = oracle.proj_rows(codes, scales, g, x, rows)
    return y.astype(np.float32)


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
