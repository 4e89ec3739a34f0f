"""CPU oracle for the NVFP4 weight-only projection (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never touches it and it
never touches the HIP library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64).  This module builds it
with gcc into ``liboracle.so`` and exposes numpy-level wrappers:

* :func:`e2m1`, :func:`e4m3`, :func:`bf16` — element decoders (closed forms),
* :func:`dequant_row` — one weight row in fp64,
* :func:`proj` / :func:`proj_rows` — y and the tolerance base S in fp64,
* :func:`check` — the acceptance test |y_gpu - y_ref| <= rtol * S.

Formats and layouts are documented at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

#: Tolerance factor of the acceptance test: |y - y_ref| <= RTOL * sum_k |x_k w_k|.
RTOL = 2e-3


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain C11, -O2, IEEE semantics kept)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", out, src, "-lm",
           "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str = LIB):
    """Load (building first if absent) and type the oracle library."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.orc_e2m1.argtypes = [ctypes.c_uint]
    lib.orc_e2m1.restype = dbl
    lib.orc_e4m3.argtypes = [ctypes.c_uint]
    lib.orc_e4m3.restype = dbl
    lib.orc_bf16.argtypes = [ctypes.c_uint16]
    lib.orc_bf16.restype = dbl
    lib.orc_dequant_row.argtypes = [vp, vp, i64, dbl, vp]
    lib.orc_dequant_row.restype = None
    lib.orc_proj_rows.argtypes = [i64, i64, i64, vp, vp, dbl, vp, vp, i64, vp, vp,
                                  ctypes.c_int]
    lib.orc_proj_rows.restype = ctypes.c_int
    lib.orc_proj.argtypes = [i64, i64, i64, vp, vp, dbl, vp, vp, vp, ctypes.c_int]
    lib.orc_proj.restype = ctypes.c_int
    lib.orc_check.argtypes = [i64, vp, vp, vp, dbl, ctypes.POINTER(dbl)]
    lib.orc_check.restype = i64
    if path == LIB:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def e2m1(code: int, lib=None) -> float:
    return (lib or load()).orc_e2m1(code)


def e4m3(byte: int, lib=None) -> float:
    return (lib or load()).orc_e4m3(byte)


def bf16(bits: int, lib=None) -> float:
    return (lib or load()).orc_bf16(bits)


def _as_u8(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint8)


def _as_u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def dequant_row(codes_row, scales_row, K: int, g: float, lib=None) -> np.ndarray:
    c, s = _as_u8(codes_row), _as_u8(scales_row)
    assert c.size == K // 2 and s.size == K // 16
    w = np.empty(K, dtype=np.float64)
    (lib or load()).orc_dequant_row(_ptr(c), _ptr(s), K, float(g), _ptr(w))
    return w


def proj_rows(codes, scales, g: float, x, rows=None, nthreads=None, lib=None):
    """y[M][len(rows)], S[M][len(rows)] in fp64 for the given weight rows.

    codes u8 [N][K/2], scales u8 [N][K/16], x bf16 bits u16 [M][K].
    rows=None evaluates every row.
    """
    c, s, xx = _as_u8(codes), _as_u8(scales), _as_u16(x)
    N = c.shape[0]
    M, K = xx.shape
    assert c.shape == (N, K // 2) and s.shape == (N, K // 16), (c.shape, s.shape, K)
    if rows is None:
        r = None
        nrows = N
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = r.size
    y = np.zeros((M, nrows), dtype=np.float64)
    S = np.zeros((M, nrows), dtype=np.float64)
    rc = (lib or load()).orc_proj_rows(M, N, K, _ptr(c), _ptr(s), float(g), _ptr(xx),
                                       None if r is None else _ptr(r), nrows,
                                       _ptr(y), _ptr(S),
                                       nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y, S


def proj(codes, scales, g: float, x, nthreads=None, lib=None):
    """Full y[M][N] and S[M][N] in fp64."""
    return proj_rows(codes, scales, g, x, None, nthreads, lib)


def check(y_ref, S, y_gpu, rtol: float = RTOL, lib=None):
    """Returns (number of failing elements, max |y-y_ref|/S)."""
    yr = np.ascontiguousarray(y_ref, dtype=np.float64)
    ss = np.ascontiguousarray(S, dtype=np.float64)
    yg = np.ascontiguousarray(y_gpu, dtype=np.float32)
    assert yr.shape == ss.shape == yg.shape, (yr.shape, ss.shape, yg.shape)
    worst = ctypes.c_double(0.0)
    bad = (lib or load()).orc_check(yr.size, _ptr(yr), _ptr(ss), _ptr(yg), float(rtol),
                                    ctypes.byref(worst))
    return int(bad), float(worst.value)
