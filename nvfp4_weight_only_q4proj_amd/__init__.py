"""Python binding of the q4proj C ABI (include/q4proj.h).

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of torch tensors, then calls the entry point of the same name in
``libq4proj.so`` on the current HIP stream.  All arithmetic runs in the HIP
kernels; there is no fallback path.  Importing this module raises if the
library has not been built (``python nvfp4_weight_only_q4proj_amd/_build.py``
or ``__graft_entry__.build()``).

The projection computed is

    y[m][n] = sum_k x[m][k] * e2m1(codes[n][k]) * e4m3(scales[n][k//16]) * g

with codes packed two per byte (element 2j in the low nibble), bf16 x,
fp32 y and fp32 global scale g.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4proj.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python nvfp4_weight_only_q4proj_amd/_build.py` (gfx950 only)")

_lib = ctypes.CDLL(LIB_PATH)

_i64, _sz, _vp, _f32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_lib.q4proj_packed_codes_bytes.argtypes = [_i64, _i64]
_lib.q4proj_packed_codes_bytes.restype = _sz
_lib.q4proj_packed_scales_bytes.argtypes = [_i64, _i64]
_lib.q4proj_packed_scales_bytes.restype = _sz
_lib.q4proj_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.q4proj_workspace_bytes.restype = _sz
_lib.q4proj_pack.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.q4proj_pack.restype = ctypes.c_int
_lib.q4proj_pack_gate_up.argtypes = [_vp, _vp, _vp, _vp, _f32, _f32, _i64, _i64, _vp, _vp, _vp]
_lib.q4proj_pack_gate_up.restype = ctypes.c_int
_lib.q4proj_unpack.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.q4proj_unpack.restype = ctypes.c_int
_PROJ_ARGS = [_vp, _vp, _f32, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]
_lib.q4proj_gemv.argtypes = _PROJ_ARGS
_lib.q4proj_gemv.restype = ctypes.c_int
_lib.q4proj_gemm.argtypes = _PROJ_ARGS
_lib.q4proj_gemm.restype = ctypes.c_int
_lib.q4proj_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.q4proj_gemm_workspace_bytes.restype = _sz
_lib.q4proj_gemv_noalloc.argtypes = [_vp, _vp, _f32, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.q4proj_gemv_noalloc.restype = ctypes.c_int
_lib.q4proj_silu_mul_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.q4proj_silu_mul_workspace_bytes.restype = _sz
_lib.q4proj_gemv_silu_mul.argtypes = _PROJ_ARGS
_lib.q4proj_gemv_silu_mul.restype = ctypes.c_int
_lib.q4proj_gemm_silu_mul.argtypes = _PROJ_ARGS
_lib.q4proj_gemm_silu_mul.restype = ctypes.c_int
_lib.q4proj_argmax_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.q4proj_argmax_workspace_bytes.restype = _sz
_lib.q4proj_gemv_argmax.argtypes = [_vp, _vp, _f32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz,
                                    _vp]
_lib.q4proj_gemv_argmax.restype = ctypes.c_int
_lib.q4proj_quantize_workspace_bytes.argtypes = [_i64, _i64]
_lib.q4proj_quantize_workspace_bytes.restype = _sz
_lib.q4proj_quantize.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.q4proj_quantize.restype = ctypes.c_int
_lib.q4proj_status_string.argtypes = [ctypes.c_int]
_lib.q4proj_status_string.restype = ctypes.c_char_p
_lib.q4proj_last_hip_error.argtypes = []
_lib.q4proj_last_hip_error.restype = ctypes.c_char_p

#: Exported symbols declared by include/q4proj.h.
SYMBOLS = ("q4proj_packed_codes_bytes", "q4proj_packed_scales_bytes", "q4proj_workspace_bytes",
           "q4proj_pack", "q4proj_pack_gate_up", "q4proj_unpack", "q4proj_gemv", "q4proj_gemm",
           "q4proj_gemm_workspace_bytes", "q4proj_gemv_noalloc",
           "q4proj_silu_mul_workspace_bytes", "q4proj_gemv_silu_mul", "q4proj_gemm_silu_mul",
           "q4proj_argmax_workspace_bytes", "q4proj_gemv_argmax",
           "q4proj_quantize_workspace_bytes", "q4proj_quantize",
           "q4proj_status_string", "q4proj_last_hip_error")

OK, EINVAL, EUNSUPPORTED, EDEVICE, EWORKSPACE, EHIP = range(6)
GEMV_MAX_M = 16


class Q4ProjError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.q4proj_status_string(status).decode()
        if status == EHIP:
            msg += ": " + _lib.q4proj_last_hip_error().decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != OK:
        raise Q4ProjError(status, where)


def library():
    """The loaded ctypes library (for callers that want the raw C ABI)."""
    return _lib


@functools.lru_cache(maxsize=4096)
def q4proj_packed_codes_bytes(N: int, K: int) -> int:
    return int(_lib.q4proj_packed_codes_bytes(N, K))


@functools.lru_cache(maxsize=4096)
def q4proj_packed_scales_bytes(N: int, K: int) -> int:
    return int(_lib.q4proj_packed_scales_bytes(N, K))


@functools.lru_cache(maxsize=4096)
def q4proj_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.q4proj_workspace_bytes(M, N, K))


@functools.lru_cache(maxsize=4096)
def q4proj_silu_mul_workspace_bytes(M: int, F: int, K: int) -> int:
    return int(_lib.q4proj_silu_mul_workspace_bytes(M, F, K))


@functools.lru_cache(maxsize=4096)
def q4proj_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.q4proj_gemm_workspace_bytes(M, N, K))


# The checks below sit on the decode path (one call per projection, ~12 us of
# GPU time each), so they use the cheap tensor queries: device indices rather
# than torch.device objects, the raw current-stream handle, and no device
# switch when the tensors are on the current device.
_SAME_DEVICE = contextlib.nullcontext()
# torch's own fast accessors (private; the public calls are the fallback)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _dev(t, name: str) -> int:
    """Index of the HIP device holding tensor t."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    d = t.get_device()
    if d < 0:
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    return d


def _guard(dev: int):
    """Make device dev current for the call (a no-op when it already is)."""
    return _SAME_DEVICE if _cur_device() == dev else torch.cuda.device(dev)


def _stream(dev: int, stream):
    """hipStream_t of `stream` (a torch stream or a raw handle), or of device
    dev's current stream."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(dev)
        stream = torch.cuda.current_stream(dev)
    return stream if isinstance(stream, int) else stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, numel: int, dev: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.get_device() != dev:
        raise ValueError(f"{name} must be on cuda:{dev}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def q4proj_pack(codes: torch.Tensor, scales: torch.Tensor, N: int, K: int,
                packed_codes: torch.Tensor, packed_scales: torch.Tensor, stream=None) -> None:
    """codes u8 [N][K/2], scales u8 [N][K/16] -> packed buffers (u8, sizes from
    q4proj_packed_*_bytes)."""
    dev = _dev(codes, "codes")
    _need(codes, "codes", torch.uint8, N * (K // 2), dev)
    _need(scales, "scales", torch.uint8, N * (K // 16), dev)
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    with _guard(dev):
        _check(_lib.q4proj_pack(codes.data_ptr(), scales.data_ptr(), N, K, packed_codes.data_ptr(),
                                packed_scales.data_ptr(), _stream(dev, stream)), "q4proj_pack")


def q4proj_pack_gate_up(gate_codes, gate_scales, up_codes, up_scales, gate_global_scale: float,
                        up_global_scale: float, F: int, K: int, packed_codes, packed_scales,
                        stream=None) -> None:
    """Separate canonical gate and up weights (u8 [F][K/2] codes, [F][K/16]
    scales, equal global scales) -> the packed fused [2F][K] gate/up weight
    (8 gate rows and 8 up rows alternating)."""
    dev = _dev(gate_codes, "gate_codes")
    for t, name in ((gate_codes, "gate_codes"), (up_codes, "up_codes")):
        _need(t, name, torch.uint8, F * (K // 2), dev)
    for t, name in ((gate_scales, "gate_scales"), (up_scales, "up_scales")):
        _need(t, name, torch.uint8, F * (K // 16), dev)
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(2 * F, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(2 * F, K), dev)
    with _guard(dev):
        _check(_lib.q4proj_pack_gate_up(gate_codes.data_ptr(), gate_scales.data_ptr(),
                                        up_codes.data_ptr(), up_scales.data_ptr(),
                                        float(gate_global_scale), float(up_global_scale), F, K,
                                        packed_codes.data_ptr(), packed_scales.data_ptr(),
                                        _stream(dev, stream)), "q4proj_pack_gate_up")


def q4proj_unpack(packed_codes: torch.Tensor, packed_scales: torch.Tensor, N: int, K: int,
                  codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    dev = _dev(packed_codes, "packed_codes")
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    _need(codes, "codes", torch.uint8, N * (K // 2), dev)
    _need(scales, "scales", torch.uint8, N * (K // 16), dev)
    with _guard(dev):
        _check(_lib.q4proj_unpack(packed_codes.data_ptr(), packed_scales.data_ptr(), N, K,
                                  codes.data_ptr(), scales.data_ptr(), _stream(dev, stream)),
               "q4proj_unpack")


_workspaces: dict = {}
_gemm_scratch: dict = {}


def _stream_handle_and_obj(dev: int, stream):
    """(raw hipStream_t, torch stream object) of `stream`, or of device dev's
    current stream when stream is None."""
    if stream is None:
        obj = torch.cuda.current_stream(dev)
        return obj.cuda_stream, obj
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream, stream
    handle = int(stream)
    return handle, torch.cuda.ExternalStream(handle, device=torch.device("cuda", dev))


def default_workspace(device, nbytes: int, stream=None):
    """A zero-filled device buffer of at least nbytes for calls on `stream`
    (default: the device's current stream) that pass no workspace.

    One buffer per (device, stream): calls on one stream run in order, so
    they can share it (each call leaves it zero-filled); calls on different
    streams get different buffers and may run concurrently.  The buffer is
    allocated and zero-filled on that stream, so the fill is ordered before
    the calls that use it, and torch's caching allocator ties the memory to
    that stream.  A call that returned an error enqueued nothing and left
    the buffer as it was; only a kernel that did not run to completion (a
    device fault, a killed process) can leave words set, and the process's
    device state is then lost anyway."""
    if nbytes <= 0:
        return None
    dev = device if isinstance(device, int) else (
        torch.device(device).index if torch.device(device).index is not None
        else torch.cuda.current_device())
    key = (dev, _stream(dev, stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        _, sobj = _stream_handle_and_obj(dev, stream)
        with torch.cuda.stream(sobj):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=torch.device("cuda", dev))
        _workspaces[key] = ws
    return ws


def gemm_scratch(device, nbytes: int, stream=None):
    """A device buffer of at least nbytes for q4proj_gemm / q4proj_gemm_silu_mul
    calls on `stream` (default: the device's current stream) that pass no
    workspace: the GEMMs stage their fp16 activations there.  Its contents
    do not matter (it is never zero-filled) and it is kept apart from the
    zero-filled default workspaces of the GEMV entry points.  One per
    (device, stream), allocated on that stream."""
    dev = device if isinstance(device, int) else (
        torch.device(device).index if torch.device(device).index is not None
        else torch.cuda.current_device())
    key = (dev, _stream(dev, stream))
    ws = _gemm_scratch.get(key)
    if ws is None or ws.numel() < nbytes:
        _, sobj = _stream_handle_and_obj(dev, stream)
        with torch.cuda.stream(sobj):
            ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device("cuda", dev))
        _gemm_scratch[key] = ws
    return ws


def gemm_staging_pays(M: int, N: int, K: int) -> bool:
    """Whether fp16 operands pay for their staging on this shape: they take
    about 8 % off the GEMM kernel's time, and the staging kernel costs about
    4 us plus its 4 bytes per activation at ~5 TB/s (MI355X, measured at
    M = 512, K = 5120: level at N = 14336, a gain at N = 17408 and above).
    The results are the same either way."""
    t_gemm = 2.0 * M * N * K / 1.0e15
    t_stage = 4.0e-6 + 4.0 * M * K / 5.0e12
    return 0.08 * t_gemm > t_stage


def _gemm_workspace(dev, workspace, M, N, K, stream):
    """The workspace a GEMM call passes: workspace=None takes the per-stream
    scratch (fp16 operands) where gemm_staging_pays, else none; False none
    (bf16 operands); a tensor is passed as given."""
    if workspace is None:
        if not gemm_staging_pays(M, N, K):
            return None
        return gemm_scratch(dev, q4proj_gemm_workspace_bytes(M, N, K), stream)
    if workspace is False:
        return None
    return workspace


def _bf16_bits(t, name):
    """A bfloat16 tensor as its 16-bit patterns (a view); int16/uint16 pass."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 (bfloat16 or 16-bit bit patterns)")
    return t


def _proj_args(name, packed_codes, packed_scales, global_scale, x, y, M, N, K, workspace,
               stream):
    """Checks of a projection call; (device, the C arguments, the tensors they
    point into)."""
    dev = _dev(x, "x")
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    x = _bf16_bits(x, "x")
    _need(x, "x", x.dtype, M * K, dev)
    _need(y, "y", torch.float32, M * N, dev)
    ws_ptr, ws_bytes = None, 0
    if name == "q4proj_gemm":
        workspace = _gemm_workspace(dev, workspace, M, N, K, stream)
    elif workspace is None and name == "q4proj_gemv":
        workspace = default_workspace(dev, q4proj_workspace_bytes(M, N, K), stream)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, workspace.numel(), dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    args = (packed_codes.data_ptr(), packed_scales.data_ptr(), float(global_scale), x.data_ptr(),
            y.data_ptr(), M, N, K, ws_ptr, ws_bytes, _stream(dev, stream))
    return dev, args, (packed_codes, packed_scales, x, y, workspace)


def _proj(fn, where, packed_codes, packed_scales, global_scale, x, y, M, N, K, workspace, stream):
    dev, args, _ = _proj_args(where, packed_codes, packed_scales, global_scale, x, y, M, N, K,
                              workspace, stream)
    with _guard(dev):
        _check(fn(*args), where)


def q4proj_gemv(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int, K: int,
                workspace=None, stream=None) -> None:
    """y[M][N] fp32 = x[M][K] bf16 . dequant(W)^T for 1 <= M <= 16."""
    _proj(_lib.q4proj_gemv, "q4proj_gemv", packed_codes, packed_scales, global_scale, x, y, M, N,
          K, workspace, stream)


def q4proj_gemv_noalloc(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int,
                        K: int, stream=None) -> None:
    """q4proj_gemv with the library's per-GPU scratch array in place of a
    workspace (allocates nothing; calls that overlap on one GPU race)."""
    dev = _dev(x, "x")
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    x = _bf16_bits(x, "x")
    _need(x, "x", x.dtype, M * K, dev)
    _need(y, "y", torch.float32, M * N, dev)
    with _guard(dev):
        _check(_lib.q4proj_gemv_noalloc(packed_codes.data_ptr(), packed_scales.data_ptr(),
                                        float(global_scale), x.data_ptr(), y.data_ptr(), M, N, K,
                                        _stream(dev, stream)), "q4proj_gemv_noalloc")


def q4proj_gemm(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int, K: int,
                workspace=None, stream=None) -> None:
    """y[M][N] fp32 = x[M][K] bf16 . dequant(W)^T for any M >= 1.
    workspace: None takes the stream's GEMM scratch (fp16 operands) on shapes
    where that pays (gemm_staging_pays) and none otherwise, False runs
    without one (bf16 operands, the same results), a uint8 tensor of
    q4proj_gemm_workspace_bytes(M, N, K) bytes is used as given."""
    _proj(_lib.q4proj_gemm, "q4proj_gemm", packed_codes, packed_scales, global_scale, x, y, M, N,
          K, workspace, stream)


def q4proj_gemv_silu_mul(packed_codes, packed_scales, global_scale: float, x, h, M: int, F: int,
                         K: int, workspace=None, stream=None) -> None:
    """h[M][F] bf16 = silu(gate) * up of the fused [2F][K] gate/up weight
    (8-row gate and up blocks alternating), 1 <= M <= 16."""
    _silu_mul(_lib.q4proj_gemv_silu_mul, "q4proj_gemv_silu_mul", packed_codes, packed_scales,
              global_scale, x, h, M, F, K, workspace, stream)


def q4proj_gemm_silu_mul(packed_codes, packed_scales, global_scale: float, x, h, M: int, F: int,
                         K: int, workspace=None, stream=None) -> None:
    """As q4proj_gemv_silu_mul for any M >= 1 (matrix-core path); workspace as
    q4proj_gemm's (N = 2F)."""
    _silu_mul(_lib.q4proj_gemm_silu_mul, "q4proj_gemm_silu_mul", packed_codes, packed_scales,
              global_scale, x, h, M, F, K, workspace, stream)


def _silu_mul_args(name, packed_codes, packed_scales, global_scale, x, h, M, F, K, workspace,
                   stream):
    dev = _dev(x, "x")
    N = 2 * F
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    x = _bf16_bits(x, "x")
    h = _bf16_bits(h, "h")
    _need(x, "x", x.dtype, M * K, dev)
    _need(h, "h", h.dtype, M * F, dev)
    ws_ptr, ws_bytes = None, 0
    if name == "q4proj_gemm_silu_mul":
        workspace = _gemm_workspace(dev, workspace, M, N, K, stream)
    elif workspace is None and name == "q4proj_gemv_silu_mul":
        workspace = default_workspace(dev, q4proj_silu_mul_workspace_bytes(M, F, K), stream)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, workspace.numel(), dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    args = (packed_codes.data_ptr(), packed_scales.data_ptr(), float(global_scale), x.data_ptr(),
            h.data_ptr(), M, F, K, ws_ptr, ws_bytes, _stream(dev, stream))
    return dev, args, (packed_codes, packed_scales, x, h, workspace)


def _silu_mul(fn, where, packed_codes, packed_scales, global_scale, x, h, M, F, K, workspace,
              stream):
    dev, args, _ = _silu_mul_args(where, packed_codes, packed_scales, global_scale, x, h, M, F,
                                  K, workspace, stream)
    with _guard(dev):
        _check(fn(*args), where)


@functools.lru_cache(maxsize=4096)
def q4proj_argmax_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.q4proj_argmax_workspace_bytes(M, N, K))


def q4proj_gemv_argmax(packed_codes, packed_scales, global_scale: float, x, y, max_val, max_idx,
                       M: int, N: int, K: int, workspace=None, stream=None) -> None:
    """Greedy argmax of each row of the logits x . dequant(W)^T (1 <= M <= 16):
    max_val float32 [M], max_idx int64 [M]; y (fp32 [M][N]) may be None."""
    dev, args, _ = _argmax_args(packed_codes, packed_scales, global_scale, x, y, max_val,
                                max_idx, M, N, K, workspace, stream)
    with _guard(dev):
        _check(_lib.q4proj_gemv_argmax(*args), "q4proj_gemv_argmax")


def _argmax_args(packed_codes, packed_scales, global_scale, x, y, max_val, max_idx, M, N, K,
                 workspace, stream):
    dev = _dev(x, "x")
    _need(packed_codes, "packed_codes", torch.uint8, q4proj_packed_codes_bytes(N, K), dev)
    _need(packed_scales, "packed_scales", torch.uint8, q4proj_packed_scales_bytes(N, K), dev)
    x = _bf16_bits(x, "x")
    _need(x, "x", x.dtype, M * K, dev)
    if y is not None:
        _need(y, "y", torch.float32, M * N, dev)
    _need(max_val, "max_val", torch.float32, M, dev)
    _need(max_idx, "max_idx", torch.int64, M, dev)
    if workspace is None:
        workspace = default_workspace(dev, q4proj_argmax_workspace_bytes(M, N, K), stream)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, workspace.numel(), dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    args = (packed_codes.data_ptr(), packed_scales.data_ptr(), float(global_scale), x.data_ptr(),
            None if y is None else y.data_ptr(), max_val.data_ptr(), max_idx.data_ptr(), M, N, K,
            ws_ptr, ws_bytes, _stream(dev, stream))
    return dev, args, (packed_codes, packed_scales, x, y, max_val, max_idx, workspace)


# ---- prepared calls ---------------------------------------------------------
# A decode loop makes the same call on the same buffers every step.  The
# prepare_* functions run the eager call's checks once and return a launcher
# that goes straight to the C entry point with its arguments already
# converted to C values: no per-call Python checks (the library still
# validates every call on the host).
_lib_raw = ctypes.CDLL(LIB_PATH)    # the same library, entry points without argtypes

# C types of the eleven arguments shared by the projection entry points
_PROJ_CTYPES = (_vp, _vp, _f32, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp)
_ARGMAX_CTYPES = (_vp, _vp, _f32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp)


class Prepared:
    """One entry point bound to fixed buffers, sizes, workspace and stream
    (the stream current at preparation when none was given).  Calling it
    enqueues the call again.  It keeps the tensors it was prepared with
    alive; they must keep their storage (no resize, no re-allocation).  The
    device they live on is made current for the call when it is not."""

    __slots__ = ("_fn", "_args", "_where", "_dev", "_keep")

    def __init__(self, name, ctypes_seq, args, dev, keep):
        self._fn = getattr(_lib_raw, name)
        self._fn.restype = ctypes.c_int
        self._args = tuple(t(a) for t, a in zip(ctypes_seq, args))
        self._where = name
        self._dev = dev
        self._keep = keep

    def __call__(self) -> None:
        if _cur_device() == self._dev:
            st = self._fn(*self._args)
        else:
            with torch.cuda.device(self._dev):
                st = self._fn(*self._args)
        if st != OK:
            raise Q4ProjError(st, self._where)


def prepare_gemv(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int, K: int,
                 workspace=None, stream=None) -> Prepared:
    """q4proj_gemv bound to these buffers (see Prepared)."""
    dev, args, keep = _proj_args("q4proj_gemv", packed_codes, packed_scales, global_scale, x, y,
                                 M, N, K, workspace, stream)
    return Prepared("q4proj_gemv", _PROJ_CTYPES, args, dev, keep)


def prepare_gemm(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int, K: int,
                 workspace=None, stream=None) -> Prepared:
    """q4proj_gemm bound to these buffers (see Prepared)."""
    dev, args, keep = _proj_args("q4proj_gemm", packed_codes, packed_scales, global_scale, x, y,
                                 M, N, K, workspace, stream)
    return Prepared("q4proj_gemm", _PROJ_CTYPES, args, dev, keep)


def prepare_gemv_silu_mul(packed_codes, packed_scales, global_scale: float, x, h, M: int, F: int,
                          K: int, workspace=None, stream=None) -> Prepared:
    """q4proj_gemv_silu_mul bound to these buffers (see Prepared)."""
    dev, args, keep = _silu_mul_args("q4proj_gemv_silu_mul", packed_codes, packed_scales,
                                     global_scale, x, h, M, F, K, workspace, stream)
    return Prepared("q4proj_gemv_silu_mul", _PROJ_CTYPES, args, dev, keep)


def prepare_gemm_silu_mul(packed_codes, packed_scales, global_scale: float, x, h, M: int, F: int,
                          K: int, workspace=None, stream=None) -> Prepared:
    """q4proj_gemm_silu_mul bound to these buffers (see Prepared)."""
    dev, args, keep = _silu_mul_args("q4proj_gemm_silu_mul", packed_codes, packed_scales,
                                     global_scale, x, h, M, F, K, workspace, stream)
    return Prepared("q4proj_gemm_silu_mul", _PROJ_CTYPES, args, dev, keep)


def prepare_gemv_noalloc(packed_codes, packed_scales, global_scale: float, x, y, M: int, N: int,
                         K: int, stream=None) -> Prepared:
    """q4proj_gemv_noalloc bound to these buffers (see Prepared)."""
    dev, args, keep = _proj_args("q4proj_gemv_noalloc", packed_codes, packed_scales, global_scale,
                                 x, y, M, N, K, None, stream)
    noalloc_args = args[:8] + args[10:]                  # no workspace arguments
    return Prepared("q4proj_gemv_noalloc", _PROJ_CTYPES[:8] + _PROJ_CTYPES[10:], noalloc_args,
                    dev, keep)


def prepare_gemv_argmax(packed_codes, packed_scales, global_scale: float, x, y, max_val, max_idx,
                        M: int, N: int, K: int, workspace=None, stream=None) -> Prepared:
    """q4proj_gemv_argmax bound to these buffers (see Prepared)."""
    dev, args, keep = _argmax_args(packed_codes, packed_scales, global_scale, x, y, max_val,
                                   max_idx, M, N, K, workspace, stream)
    return Prepared("q4proj_gemv_argmax", _ARGMAX_CTYPES, args, dev, keep)


def q4proj_quantize_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.q4proj_quantize_workspace_bytes(N, K))


def q4proj_quantize(w, N: int, K: int, codes: torch.Tensor, scales: torch.Tensor,
                    global_scale: torch.Tensor, workspace=None, stream=None) -> None:
    """bf16 w [N][K] -> codes u8 [N][K/2], scales u8 [N][K/16], global_scale
    (a one-element float32 device tensor)."""
    w = _bf16_bits(w, "w")
    dev = _dev(w, "w")
    _need(w, "w", w.dtype, N * K, dev)
    _need(codes, "codes", torch.uint8, N * (K // 2), dev)
    _need(scales, "scales", torch.uint8, N * (K // 16), dev)
    _need(global_scale, "global_scale", torch.float32, 1, dev)
    if workspace is None:
        # a temporary allocated on the stream the kernels run on, so that the
        # caching allocator does not hand it out again before they are done
        _, sobj = _stream_handle_and_obj(dev, stream)
        with torch.cuda.stream(sobj):
            workspace = torch.empty(q4proj_quantize_workspace_bytes(N, K), dtype=torch.uint8,
                                    device=torch.device("cuda", dev))
    _need(workspace, "workspace", torch.uint8, workspace.numel(), dev)
    with _guard(dev):
        _check(_lib.q4proj_quantize(w.data_ptr(), N, K, codes.data_ptr(), scales.data_ptr(),
                                    global_scale.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), _stream(dev, stream)), "q4proj_quantize")


def quantize_weight(w, N: int, K: int, stream=None):
    """Allocate canonical codes/scales and a device global scale on w.device
    (on the stream the quantizer runs on) and fill them with q4proj_quantize."""
    dev = w.device
    _, sobj = _stream_handle_and_obj(_dev(w, "w"), stream)
    with torch.cuda.stream(sobj):
        codes = torch.empty(N * (K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty(N * (K // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
    q4proj_quantize(w, N, K, codes, scales, g, stream=stream)
    return codes, scales, g


def pack_gate_up_weight(gate_codes, gate_scales, up_codes, up_scales, gate_global_scale: float,
                        up_global_scale: float, F: int, K: int, stream=None):
    """Allocate the packed fused gate/up buffers on gate_codes.device and fill
    them with q4proj_pack_gate_up."""
    _, sobj = _stream_handle_and_obj(_dev(gate_codes, "gate_codes"), stream)
    with torch.cuda.stream(sobj):
        pc = torch.empty(q4proj_packed_codes_bytes(2 * F, K), dtype=torch.uint8,
                         device=gate_codes.device)
        ps = torch.empty(q4proj_packed_scales_bytes(2 * F, K), dtype=torch.uint8,
                         device=gate_codes.device)
    q4proj_pack_gate_up(gate_codes, gate_scales, up_codes, up_scales, gate_global_scale,
                        up_global_scale, F, K, pc, ps, stream)
    return pc, ps


def pack_weight(codes: torch.Tensor, scales: torch.Tensor, N: int, K: int, stream=None):
    """Allocate packed buffers on codes.device (on the stream the swizzle runs
    on) and fill them with q4proj_pack."""
    _, sobj = _stream_handle_and_obj(_dev(codes, "codes"), stream)
    with torch.cuda.stream(sobj):
        pc = torch.empty(q4proj_packed_codes_bytes(N, K), dtype=torch.uint8, device=codes.device)
        ps = torch.empty(q4proj_packed_scales_bytes(N, K), dtype=torch.uint8, device=codes.device)
    q4proj_pack(codes, scales, N, K, pc, ps, stream)
    return pc, ps
