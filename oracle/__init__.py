"""CPU oracle for the NVFP4 weight-only projection (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never touches it and it
never touches the HIP library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64).  ``__graft_entry__.build()``
compiles it with gcc into ``liboracle.so`` (this module never compiles
anything itself: it is loaded by processes that already use the GPU, which
must not start other programs); the module exposes numpy-level wrappers:

* :func:`e2m1`, :func:`e4m3`, :func:`bf16` — element decoders (closed forms),
* :func:`dequant_row` — one weight row in fp64,
* :func:`proj` / :func:`proj_rows` — y and the tolerance base S in fp64,
* :func:`check` — the acceptance test |y_gpu - y_ref| <= rtol * S,
* :func:`argmax_check` — the acceptance test of a greedy argmax (index and
  value) over logits rows,
* :func:`quantize` / :func:`quant_global_scale` — the NVFP4 quantizer
  (bf16 weights -> codes, e4m3 block scales, global scale), every rounding
  decision taken exactly (nearest value to the exact quotient, ties to even),
* :func:`silu_mul_cols` / :func:`check_bf16` — the fused gate/up projection
  h = silu(gate) * up on a weight whose gate and up rows are interleaved in
  groups of 8, its error allowance, and the bf16 acceptance test.

Formats and layouts are documented at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB_PLAIN = os.path.join(_HERE, "liboracle.so")
#: The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
#: (errors fatal).  Loading it needs the ASan runtime preloaded into the
#: process; the CPU test of the sanitizer leg starts such processes.
LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
#: Set to 1 in the environment to load (and build mutants as) the sanitized
#: library.
SANITIZE_ENV = "Q4P_SANITIZED_ORACLE"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def sanitized() -> bool:
    return os.environ.get(SANITIZE_ENV) == "1"


LIB = LIB_SAN if sanitized() else LIB_PLAIN

#: Tolerance factor of the acceptance test: |y - y_ref| <= RTOL * sum_k |x_k w_k|.
RTOL = 2e-3


def build(src: str = SRC, out: str = LIB, sanitize: bool | None = None) -> str:
    """Compile the oracle with gcc (plain C11, -O2, IEEE semantics kept);
    with ``sanitize`` (default: the environment switch) under ASan and UBSan.
    The sanitizers change no floating-point semantics."""
    if sanitize is None:
        sanitize = sanitized()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra"]
    if sanitize:
        cmd += SANITIZE_FLAGS
    cmd += ["-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str = LIB):
    """Load and type the oracle library (built by ``build()``)."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python __graft_entry__.py build` "
                          "(or oracle.build()) before loading the oracle")
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
    lib.orc_silu_mul.argtypes = [i64, vp, vp, vp]
    lib.orc_silu_mul.restype = None
    lib.orc_silu_mul_bound.argtypes = [i64, vp, vp, vp, vp, dbl, vp]
    lib.orc_silu_mul_bound.restype = None
    lib.orc_check_bf16.argtypes = [i64, vp, vp, vp, ctypes.POINTER(dbl)]
    lib.orc_check_bf16.restype = i64
    lib.orc_argmax_check.argtypes = [i64, i64, vp, vp, dbl, vp, vp]
    lib.orc_argmax_check.restype = i64
    lib.orc_quant_scale.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.orc_quant_scale.restype = ctypes.c_uint
    lib.orc_quant_code.argtypes = [ctypes.c_float, ctypes.c_uint, ctypes.c_float]
    lib.orc_quant_code.restype = ctypes.c_uint
    lib.orc_quant_global_scale.argtypes = [i64, vp]
    lib.orc_quant_global_scale.restype = ctypes.c_float
    lib.orc_quantize.argtypes = [i64, i64, vp, ctypes.c_float, vp, vp]
    lib.orc_quantize.restype = None
    if path == LIB:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    """The CPU cores this process may run on (its affinity set), which on a
    shared host can be fewer than os.cpu_count()."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


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


# ---- fused gate/up + silu(gate) * up --------------------------------------

def gate_up_rows(F: int):
    """Rows of the fused [2F][K] weight holding gate row f and up row f
    (interleaved in groups of 8: gate rows 8p.. at 16p.., up rows 8 later)."""
    f = np.arange(F, dtype=np.int64)
    gate = 16 * (f // 8) + f % 8
    return gate, gate + 8


def silu_mul(gate, up, lib=None) -> np.ndarray:
    """h = silu(gate) * up in fp64, elementwise."""
    a = np.ascontiguousarray(gate, dtype=np.float64)
    b = np.ascontiguousarray(up, dtype=np.float64)
    assert a.shape == b.shape
    h = np.empty_like(a)
    (lib or load()).orc_silu_mul(a.size, _ptr(a), _ptr(b), _ptr(h))
    return h


def silu_mul_cols(codes, scales, g: float, x, F: int, cols=None, nthreads=None, lib=None):
    """h[M][len(cols)] = silu(gate) * up in fp64 for output columns `cols` of
    the fused projection (codes/scales of the interleaved [2F][K] weight), and
    the allowance bound[M][len(cols)] of the fp32 path before its bf16
    rounding.  cols=None evaluates every column."""
    lib = lib or load()
    grow, urow = gate_up_rows(F)
    if cols is not None:
        c = np.asarray(cols, dtype=np.int64)
        grow, urow = grow[c], urow[c]
    a, Sa = proj_rows(codes, scales, g, x, grow, nthreads, lib)
    b, Sb = proj_rows(codes, scales, g, x, urow, nthreads, lib)
    h = silu_mul(a, b, lib)
    bound = np.empty_like(h)
    lib.orc_silu_mul_bound(h.size, _ptr(a), _ptr(b), _ptr(Sa), _ptr(Sb), float(RTOL), _ptr(bound))
    return h, bound


def silu_mul_separate(gate_codes, gate_scales, up_codes, up_scales, g: float, x, nthreads=None,
                      lib=None):
    """h[M][F] = silu(gate) * up in fp64 from two separate [F][K] weights with
    the one global scale g (the plain definition of the fused projection,
    no row interleave), and the allowance bound of the fp32 path before its
    bf16 rounding."""
    lib = lib or load()
    a, Sa = proj(gate_codes, gate_scales, g, x, nthreads, lib)
    b, Sb = proj(up_codes, up_scales, g, x, nthreads, lib)
    h = silu_mul(a, b, lib)
    bound = np.empty_like(h)
    lib.orc_silu_mul_bound(h.size, _ptr(a), _ptr(b), _ptr(Sa), _ptr(Sb), float(RTOL), _ptr(bound))
    return h, bound


def check_bf16(h_ref, bound, h_gpu_bits, lib=None):
    """Returns (number of failing elements, max |h-h_ref| / allowance)."""
    hr = np.ascontiguousarray(h_ref, dtype=np.float64)
    bd = np.ascontiguousarray(bound, dtype=np.float64)
    hg = np.ascontiguousarray(h_gpu_bits, dtype=np.uint16)
    assert hr.shape == bd.shape == hg.shape, (hr.shape, bd.shape, hg.shape)
    worst = ctypes.c_double(0.0)
    bad = (lib or load()).orc_check_bf16(hr.size, _ptr(hr), _ptr(bd), _ptr(hg), ctypes.byref(worst))
    return int(bad), float(worst.value)


def quant_global_scale(w_bits, lib=None) -> float:
    """g = amax / 2688 in fp32 (1 for an all-zero tensor) of bf16 bit patterns."""
    w = _as_u16(w_bits)
    return float((lib or load()).orc_quant_global_scale(w.size, _ptr(w)))


def quantize(w_bits, N: int, K: int, g=None, rows=None, lib=None):
    """Quantise bf16 W [N][K] (bit patterns) -> (codes u8 [R][K/2], scales u8
    [R][K/16], g) for rows `rows` (default all; R = len(rows)).  g defaults to
    the tensor's global scale."""
    lib = lib or load()
    w = _as_u16(w_bits).reshape(N, K)
    if g is None:
        g = quant_global_scale(w, lib)
    if rows is not None:
        w = np.ascontiguousarray(w[np.asarray(rows, dtype=np.int64)])
    R = w.shape[0]
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 16), dtype=np.uint8)
    lib.orc_quantize(R, K, _ptr(w), float(g), _ptr(codes), _ptr(scales))
    return codes, scales, float(g)


def argmax_check(y_ref, S, idx, val, rtol: float = RTOL, lib=None) -> int:
    """Rows whose (index, value) is not an acceptable greedy argmax of the
    exact logits y_ref [M][N] (tolerance bases S); returns the count."""
    yr = np.ascontiguousarray(y_ref, dtype=np.float64)
    sr = np.ascontiguousarray(S, dtype=np.float64)
    M, N = yr.shape
    ix = np.ascontiguousarray(idx, dtype=np.int64).reshape(M)
    vv = np.ascontiguousarray(val, dtype=np.float32).reshape(M)
    return int((lib or load()).orc_argmax_check(M, N, _ptr(yr), _ptr(sr), float(rtol), _ptr(ix),
                                                _ptr(vv)))

