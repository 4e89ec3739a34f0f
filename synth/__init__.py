"""Seeded synthetic inputs for the NVFP4 projection.

The one module that both the HIP path and the CPU oracle receive data from.
It holds random-number generation and *encoders* only (see ``synth.c``); it
decodes nothing and computes no projection.

Workloads (seed = workload index; every tensor has its own stream):

====  =====================================================================
tiny  M=1, K=256, N=512; codes uniform over the 16 e2m1 codes, block scales
      e4m3(|N(0,0.5)| + 0.01), g = 1.0, x ~ N(0,1) bf16.          (seed 0)
dec   M=1 decode on a 27B-style dense MLP: gate/up K=5120 N=17408, down
      K=17408 N=5120; weights bf16 N(0,0.02), two-level NVFP4.    (seed 1)
mtp   M=7 (6 drafts + 1) on the decode workload's weight bytes.   (seed 2, x)
pre   M=512 prefill chunk: qkv K=5120 N=14336 (seed 3), gate/up = the decode
      workload's gate/up bytes.                                    (seed 3, x)
lmh   M=1: lm-head K=5120 N=248320, 4B-model up K=2560 N=9216 and down
      K=9216 N=2560.                                              (seed 4)
====  =====================================================================
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "synth.c")
LIB_PLAIN = os.path.join(_HERE, "libsynth.so")
#: The same source under AddressSanitizer and UndefinedBehaviorSanitizer,
#: loaded instead of the plain library when the oracle's sanitizer switch
#: (Q4P_SANITIZED_ORACLE=1) is set; the ASan runtime must be preloaded.
LIB_SAN = os.path.join(_HERE, "libsynth_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]
LIB = LIB_SAN if os.environ.get("Q4P_SANITIZED_ORACLE") == "1" else LIB_PLAIN

# stream ids
STREAM_X = 100        # + matrix index
STREAM_W = 200        # + matrix index
STREAM_C0_CODES = 300
STREAM_C0_SCALES = 301

WEIGHT_STD = 0.02


def build(src: str = SRC, out: str = LIB, sanitize: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra"]
    if sanitize or out == LIB_SAN:
        cmd += SANITIZE_FLAGS
    cmd += ["-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load():
    """Load and type the generator library (built by ``build()``; this module
    never compiles anything itself, since GPU processes load it and must not
    start other programs)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is missing: run `python __graft_entry__.py build` "
                          "(or synth.build()) first")
    lib = ctypes.CDLL(LIB)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.syn_u64.argtypes = [u64, u64, u64]
    lib.syn_u64.restype = u64
    lib.syn_normal.argtypes = [u64, u64, u64]
    lib.syn_normal.restype = dbl
    lib.syn_normal_bf16.argtypes = [u64, u64, dbl, i64, i64, vp]
    lib.syn_normal_bf16.restype = None
    lib.syn_normal_bf16_amax.argtypes = [u64, u64, dbl, i64, i64]
    lib.syn_normal_bf16_amax.restype = dbl
    lib.syn_global_scale.argtypes = [dbl]
    lib.syn_global_scale.restype = ctypes.c_float
    lib.syn_quantize_rows.argtypes = [u64, u64, dbl, i64, i64, i64, ctypes.c_float, vp, vp]
    lib.syn_quantize_rows.restype = None
    lib.syn_uniform_codes.argtypes = [u64, u64, i64, i64, vp]
    lib.syn_uniform_codes.restype = None
    lib.syn_abs_normal_e4m3.argtypes = [u64, u64, dbl, dbl, i64, i64, vp]
    lib.syn_abs_normal_e4m3.restype = None
    lib.syn_encode_bf16.argtypes = [dbl]
    lib.syn_encode_bf16.restype = ctypes.c_uint16
    lib.syn_encode_e4m3.argtypes = [dbl]
    lib.syn_encode_e4m3.restype = ctypes.c_uint8
    lib.syn_encode_e2m1.argtypes = [dbl]
    lib.syn_encode_e2m1.restype = ctypes.c_uint
    _lib = lib
    return lib


def _threads(threads):
    return max(1, threads or min(os.cpu_count() or 1, 16))


def _chunks(total: int, parts: int):
    parts = max(1, min(parts * 4, total)) if total > 0 else 1
    return [(total * i // parts, total * (i + 1) // parts) for i in range(parts)]


def normal_bf16(seed: int, stream: int, count: int, std: float = 1.0, threads=None):
    """bf16 bit patterns of std * N(0,1) draws [0, count)."""
    lib = load()
    out = np.empty(count, dtype=np.uint16)
    base = out.ctypes.data

    def work(r):
        a, b = r
        if b > a:
            lib.syn_normal_bf16(seed, stream, std, a, b - a, base + 2 * a)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(work, _chunks(count, _threads(threads))))
    return out


def x_bf16(seed: int, stream: int, M: int, K: int, threads=None) -> np.ndarray:
    """Activations x[M][K] ~ N(0,1) as bf16 bit patterns."""
    return normal_bf16(seed, stream, M * K, 1.0, threads).reshape(M, K)


@dataclass
class Matrix:
    """An NVFP4 weight in canonical layout: codes u8 [N][K/2] (element 2j in
    the low nibble), e4m3 scales u8 [N][K/16], fp32 global scale g."""
    name: str
    N: int
    K: int
    codes: np.ndarray
    scales: np.ndarray
    g: float


def nvfp4_normal_matrix(seed: int, stream: int, N: int, K: int, name: str = "w",
                        std: float = WEIGHT_STD, threads=None) -> Matrix:
    """Two-level NVFP4 quantisation of a bf16 N(0, std) [N][K] matrix."""
    assert K % 16 == 0
    lib = load()
    nt = _threads(threads)
    total = N * K
    with ThreadPoolExecutor(nt) as ex:
        amaxes = list(ex.map(lambda r: lib.syn_normal_bf16_amax(seed, stream, std, r[0], r[1] - r[0])
                             if r[1] > r[0] else 0.0, _chunks(total, nt)))
    g = float(lib.syn_global_scale(max(amaxes)))
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    cb, sb = codes.ctypes.data, scales.ctypes.data

    def work(r):
        a, b = r
        if b > a:
            lib.syn_quantize_rows(seed, stream, std, K, a, b, g,
                                  cb + a * (K // 2), sb + a * (K // 16))

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(work, _chunks(N, nt)))
    return Matrix(name, N, K, codes, scales, g)


def uniform_code_matrix(seed: int, N: int, K: int, name: str = "tiny") -> Matrix:
    """Codes uniform over all 16 e2m1 codes, scales e4m3(|N(0,0.5)| + 0.01), g = 1."""
    lib = load()
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    lib.syn_uniform_codes(seed, STREAM_C0_CODES, 0, codes.size, codes.ctypes.data)
    lib.syn_abs_normal_e4m3(seed, STREAM_C0_SCALES, 0.5, 0.01, 0, scales.size,
                            scales.ctypes.data)
    return Matrix(name, N, K, codes, scales, 1.0)


@dataclass
class Case:
    """One projection call: y[M][N] = x[M][K] · dequant(matrix)^T."""
    workload: str
    name: str
    M: int
    matrix: Matrix
    x: np.ndarray

    @property
    def N(self):
        return self.matrix.N

    @property
    def K(self):
        return self.matrix.K


#: name -> (seed, M, [(matrix name, weight seed, matrix index, N, K)])
WORKLOADS = {
    "tiny": (0, 1, [("tiny", 0, 0, 512, 256)]),
    "dec": (1, 1, [("gate_up", 1, 0, 17408, 5120), ("down", 1, 1, 5120, 17408)]),
    "mtp": (2, 7, [("gate_up", 1, 0, 17408, 5120), ("down", 1, 1, 5120, 17408)]),
    "pre": (3, 512, [("qkv", 3, 0, 14336, 5120), ("gate_up", 1, 0, 17408, 5120)]),
    "lmh": (4, 1, [("lm_head", 4, 0, 248320, 5120), ("up_4b", 4, 1, 9216, 2560),
                   ("down_4b", 4, 2, 2560, 9216)]),
    # the MLP's gate and up weights as one fused [2F][K] NVFP4 weight (one
    # global scale for both), F = 17408
    "mlp": (5, 1, [("gate_up_fused", 1, 2, 34816, 5120)]),
}

#: workload names in listing order
WORKLOAD_ORDER = ["tiny", "dec", "mtp", "pre", "lmh", "mlp"]

_matrix_cache: dict = {}


def matrix(wseed: int, index: int, N: int, K: int, name: str, cache: bool = True,
           threads=None) -> Matrix:
    key = (wseed, index, N, K)
    if cache and key in _matrix_cache:
        return _matrix_cache[key]
    if wseed == 0:
        m = uniform_code_matrix(0, N, K, name)
    else:
        m = nvfp4_normal_matrix(wseed, STREAM_W + index, N, K, name, threads=threads)
    if cache:
        _matrix_cache[key] = m
    return m


def workload_cases(name: str, only=None, cache: bool = True, threads=None):
    """Full-size cases of one workload (optionally only the named matrices)."""
    seed, M, mats = WORKLOADS[name]
    cases = []
    for j, (mname, wseed, index, N, K) in enumerate(mats):
        if only is not None and mname not in only:
            continue
        mat = matrix(wseed, index, N, K, mname, cache, threads)
        x = x_bf16(seed, STREAM_X + j, M, K, threads)
        cases.append(Case(name, mname, M, mat, x))
    return cases


def clear_cache():
    _matrix_cache.clear()
