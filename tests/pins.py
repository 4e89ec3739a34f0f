"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises ``AssertionError`` when the oracle disagrees with:

* the OCP e2m1 and e4m3 tables (``tests/golden``),
* ``torch.float8_e4m3fn`` and ``torch.bfloat16`` decoding (library routines),
* exact integer arithmetic on tiny dyadic inputs (brute force),
* closed-form special cases (one-hot activations) and invariants.

The pins never call the oracle's own decoders to build expected values, so a
plausible mistake in the oracle (a swapped nibble, a wrong exponent bias, a
dropped term, a transposed operand) fails at least one of them —
``test_oracle_mutants.py`` plants such mistakes and checks exactly that.
"""
from __future__ import annotations

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---- independent decoders -------------------------------------------------

def golden_e2m1():
    """code -> value from the OCP MX fixture."""
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            table[int(parts[0], 16)] = float(parts[-1])
    assert sorted(table) == list(range(16))
    return table


def golden_e4m3_landmarks():
    out = {}
    with open(os.path.join(GOLDEN, "e4m3_ocp_ofp8_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, v = line.split()
            out[int(b, 16)] = float(v)
    return out


def torch_e4m3_table() -> np.ndarray:
    """All 256 e4m3 encodings decoded by torch.float8_e4m3fn (fp64)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def independent_dequant(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """W[N][K] in fp64 from the golden e2m1 table and torch's e4m3 decode."""
    e2 = np.array([golden_e2m1()[c] for c in range(16)], dtype=np.float64)
    e4 = torch_e4m3_table()
    N = codes.shape[0]
    K = codes.shape[1] * 2
    q = np.empty((N, K), dtype=np.float64)
    q[:, 0::2] = e2[codes & 0x0F]
    q[:, 1::2] = e2[codes >> 4]
    s = np.repeat(e4[scales], 16, axis=1)
    return q * s * np.float64(g)


# ---- tiny dyadic inputs for the exact check ---------------------------------

def tiny_inputs(M, N, K, seed, x_floor=2.0 ** -20, nan_free=True):
    """Random codes over all 16, random finite e4m3 scales, bf16 N(0,1) x with
    |x| < 2^3 and every |x| < x_floor set to 0."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    if nan_free:
        scales[(scales & 0x7F) == 0x7F] = 0x7E
    xf = rng.standard_normal((M, K))
    xf = np.clip(xf, -7.9, 7.9)
    xbits = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xv = torch_bf16(xbits)
    xbits = np.where(np.abs(xv) < x_floor, np.uint16(0), xbits).astype(np.uint16)
    return codes, scales, xbits


def exact_projection(codes, scales, g, xbits):
    """Exact y as Python Fractions, by integer arithmetic.

    x has 8 significant bits and |x| >= 2^-20 (or 0), so x * 2^27 is an integer;
    q*s is a multiple of 2^-10, so q*s * 2^10 is an integer; every product is an
    integer multiple of 2^-37 below 2^52 and a K <= 256 sum stays below 2^61.
    """
    xv = torch_bf16(xbits)
    xi = np.rint(xv * 2.0 ** 27).astype(np.int64)
    assert np.array_equal(xi.astype(np.float64) * 2.0 ** -27, xv), "x not on the 2^-27 grid"
    w = independent_dequant(codes, scales, 1.0)
    wi = np.rint(w * 2.0 ** 10).astype(np.int64)
    assert np.array_equal(wi.astype(np.float64) * 2.0 ** -10, w)
    K = xbits.shape[1]
    assert K <= 256
    yi = xi @ wi.T                                  # exact in int64 (< 2^61)
    gf = Fraction(g)
    return [[Fraction(int(v), 2 ** 37) * gf for v in row] for row in yi]


# ---- pins -----------------------------------------------------------------

def pin_e2m1_table(lib):
    table = golden_e2m1()
    for c in range(16):
        v = oracle.e2m1(c, lib)
        assert v == table[c] and math.copysign(1, v) == math.copysign(1, table[c]), (c, v)


def pin_e4m3_torch(lib):
    ref = torch_e4m3_table()
    for b in range(256):
        v = oracle.e4m3(b, lib)
        if math.isnan(ref[b]):
            assert math.isnan(v), (b, v)
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), (b, v, ref[b])


def pin_e4m3_landmarks(lib):
    for b, want in golden_e4m3_landmarks().items():
        v = oracle.e4m3(b, lib)
        if math.isnan(want):
            assert math.isnan(v), (b, v)
        else:
            assert v == want and math.copysign(1, v) == math.copysign(1, want), (b, v, want)


def pin_bf16_torch(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)     # every pattern
    ref = torch_bf16(bits)
    for b, r in zip(bits, ref):
        v = oracle.bf16(int(b), lib)
        if math.isnan(r):
            assert math.isnan(v)
        else:
            assert v == r, (hex(int(b)), v, r)


def pin_dequant_rows(lib):
    """Row dequantisation equals the independently decoded W, bit for bit."""
    rng = np.random.default_rng(11)
    N, K = 9, 96
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    for g in (1.0, 2.0 ** -10, float(np.float32(4.4531e-05))):
        W = independent_dequant(codes, scales, g)
        for n in range(N):
            w = oracle.dequant_row(codes[n], scales[n], K, g, lib)
            same = (w == W[n]) | (np.isnan(w) & np.isnan(W[n]))
            assert same.all(), (n, g, np.nonzero(~same))


SHAPES_T4 = [(M, N, K) for M in (1, 2, 7, 16, 33) for N in (1, 16, 17, 64)
             for K in (16, 32, 48, 256)]


def pin_exact_tiny(lib, shapes=None, seed0=100):
    """fp64 projection on tiny dyadic inputs.

    Strict inputs (|x| >= 2^-8, power-of-two g): every partial sum has at most
    48 significant bits, so the fp64 oracle must equal the exact value bit for
    bit.  General inputs (|x| >= 2^-20, any fp32 g): within the fp64
    summation bound K * 2^-53 * S of the correctly rounded exact value.
    """
    shapes = shapes or SHAPES_T4
    for i, (M, N, K) in enumerate(shapes):
        for strict in (True, False):
            codes, scales, xb = tiny_inputs(M, N, K, seed0 + 2 * i + strict,
                                            x_floor=2.0 ** -8 if strict else 2.0 ** -20)
            for g in ((1.0, 2.0 ** -10) if strict else (float(np.float32(3.3e-5)),)):
                y, S = oracle.proj(codes, scales, g, xb, nthreads=2, lib=lib)
                ex = exact_projection(codes, scales, g, xb)
                for m in range(M):
                    for n in range(N):
                        e = float(ex[m][n])
                        if strict:
                            assert y[m, n] == e, (M, N, K, m, n, y[m, n], e)
                        else:
                            assert abs(y[m, n] - e) <= K * 2.0 ** -53 * S[m, n] + 1e-300, \
                                (M, N, K, m, n, y[m, n], e)


def pin_exact_tiny_fast(lib):
    pin_exact_tiny(lib, [(1, 17, 48), (7, 16, 256), (33, 5, 32), (2, 64, 16)], seed0=900)


def pin_abs_sum(lib):
    """S equals sum |x * w| computed independently (fp64, same order of terms
    does not matter at this size: all terms are exact and non-negative)."""
    codes, scales, xb = tiny_inputs(3, 8, 64, 5)
    W = independent_dequant(codes, scales, 0.5)
    X = torch_bf16(xb)
    y, S = oracle.proj(codes, scales, 0.5, xb, lib=lib)
    S_ref = np.abs(X) @ np.abs(W).T
    assert np.allclose(S, S_ref, rtol=1e-14, atol=0), (S, S_ref)
    assert (S >= np.abs(y)).all()


def pin_one_hot(lib):
    """x = e_k returns exactly the dequantised column W[:, k] (closed form)."""
    rng = np.random.default_rng(3)
    N, K = 24, 64
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    g = float(np.float32(0.37))
    W = independent_dequant(codes, scales, g)
    one = 0x3F80                                   # bf16 bits of 1.0
    x = np.zeros((K, K), dtype=np.uint16)
    x[np.arange(K), np.arange(K)] = one
    y, S = oracle.proj(codes, scales, g, x, lib=lib)
    assert np.array_equal(y, W.T), "one-hot rows do not return the dequantised columns"
    assert np.array_equal(S, np.abs(W.T))


def pin_invariants(lib):
    codes, scales, xb = tiny_inputs(5, 12, 80, 21)
    g = 0.75
    y, S = oracle.proj(codes, scales, g, xb, lib=lib)
    # y(-x) = -y(x): flip the bf16 sign bit
    yn, _ = oracle.proj(codes, scales, g, xb ^ np.uint16(0x8000), lib=lib)
    assert np.array_equal(yn, -y)
    # g -> 2g doubles y exactly
    y2, _ = oracle.proj(codes, scales, 2 * g, xb, lib=lib)
    assert np.array_equal(y2, 2 * y)
    # permuting W's rows permutes y's columns
    perm = np.random.default_rng(1).permutation(codes.shape[0])
    yp, _ = oracle.proj(codes[perm], scales[perm], g, xb, lib=lib)
    assert np.array_equal(yp, y[:, perm])
    # x = 0 gives y = 0 and S = 0
    y0, S0 = oracle.proj(codes, scales, g, np.zeros_like(xb), lib=lib)
    assert not y0.any() and not S0.any()
    # a zero scale block contributes nothing: same as zeroing its codes
    sc = scales.copy()
    sc[3, 2] = 0
    cz = codes.copy()
    cz[3, 2 * 8:3 * 8] = 0
    ya, _ = oracle.proj(codes, sc, g, xb, lib=lib)
    yb, _ = oracle.proj(cz, scales, g, xb, lib=lib)
    assert np.array_equal(ya[:, 3], yb[:, 3])
    # every output only depends on its own row: evaluating a row subset agrees
    rows = np.array([7, 0, 11, 7])
    yr, Sr = oracle.proj_rows(codes, scales, g, xb, rows, lib=lib)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(Sr, S[:, rows])


def pin_nan_scale(lib):
    """A NaN scale makes its row's outputs NaN (NaN * anything), others stay finite."""
    codes, scales, xb = tiny_inputs(3, 6, 48, 8)
    scales[2, 1] = 0x7F
    scales[4, 0] = 0xFF
    y, S = oracle.proj(codes, scales, 1.0, xb, lib=lib)
    assert np.isnan(y[:, 2]).all() and np.isnan(y[:, 4]).all()
    assert np.isfinite(np.delete(y, [2, 4], axis=1)).all()


def pin_check(lib):
    """The acceptance test's semantics."""
    yref = np.array([1.0, 0.0, np.nan, 5.0, -2.0, 0.0])
    S = np.array([10.0, 0.0, 1.0, 1.0, 1.0, 3.0])
    ok = np.array([1.0 + 0.0199, 0.0, np.nan, 5.0 - 0.00199, -2.0, 0.0059], dtype=np.float32)
    bad, worst = oracle.check(yref, S, ok, lib=lib)
    assert bad == 0, bad
    assert 0.0019 < worst <= 0.002, worst
    for i, v in [(0, 1.0 + 0.021), (1, 1e-30), (2, 1.0), (3, np.inf), (4, -2.0025),
                 (5, 0.0061)]:
        t = ok.copy()
        t[i] = v
        bad, _ = oracle.check(yref, S, t, lib=lib)
        assert bad == 1, (i, v, bad)


def pin_synth_roundtrip(lib):
    """The generator's quantised bytes dequantise back near the bf16 weights it
    drew: |w - dequant(q)| <= half an e2m1 step at the block scale (a check of
    the quantiser against the oracle's decoders, on a small matrix)."""
    m = synth.nvfp4_normal_matrix(77, 1, 8, 64, threads=1)
    wbits = synth.normal_bf16(77, 1, 8 * 64, std=synth.WEIGHT_STD, threads=1).reshape(8, 64)
    w = torch_bf16(wbits)
    for n in range(8):
        d = oracle.dequant_row(m.codes[n], m.scales[n], 64, m.g, lib)
        s = np.repeat([oracle.e4m3(int(b), lib) for b in m.scales[n]], 16) * m.g
        # largest e2m1 gap is 2 (between 4 and 6); clamp at 6 adds at most (6.x-6)
        assert (np.abs(w[n] - d) <= 1.0 * s + 1e-12).all()


# ---- fused gate/up + silu(gate) * up --------------------------------------

def pin_silu_mul_torch(lib):
    """silu(gate) * up against torch.nn.functional.silu (a library routine) in
    fp64, over magnitudes from 1e-6 to 800 of both signs, and two closed
    forms: silu(0) = 0 and silu(1) = 1 / (1 + 1/e)."""
    rng = np.random.default_rng(5)
    mag = 10.0 ** rng.uniform(-6, np.log10(800.0), 4000)
    gate = mag * rng.choice([-1.0, 1.0], mag.size)
    up = rng.normal(0.0, 3.0, gate.size)
    h = oracle.silu_mul(gate, up, lib)
    ref = (torch.nn.functional.silu(torch.from_numpy(gate)) * torch.from_numpy(up)).numpy()
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300), np.max(np.abs(h - ref))
    h0 = oracle.silu_mul(np.array([0.0, 1.0, -1.0]), np.array([7.0, 1.0, 1.0]), lib)
    assert h0[0] == 0.0
    assert abs(h0[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(h0[2] + 1.0 / (1.0 + math.e)) < 1e-15


def _interleave8(gate, up):
    """Stack [F][W] gate and up row blocks as the fused weight: groups of 8
    gate rows then 8 up rows (F a multiple of 8)."""
    F, W = gate.shape
    return np.stack([gate.reshape(F // 8, 8, W), up.reshape(F // 8, 8, W)], axis=1).reshape(2 * F, W)


def pin_silu_mul_fused_rows(lib):
    """The fused projection's row selection: separate gate and up matrices,
    interleaved here with a reshape, projected by the fused path, against the
    plain projections of the separate matrices and torch's silu."""
    F, K, M = 48, 96, 3
    mg = synth.nvfp4_normal_matrix(81, 1, F, K, threads=1)
    mu = synth.nvfp4_normal_matrix(81, 2, F, K, threads=1)
    x = synth.x_bf16(81, 3, M, K, threads=1)
    codes = _interleave8(mg.codes, mu.codes)
    scales = _interleave8(mg.scales, mu.scales)
    g = 0.75                                       # one global scale for both halves
    h, _ = oracle.silu_mul_cols(codes, scales, g, x, F, lib=lib)
    a, _ = oracle.proj(mg.codes, mg.scales, g, x, lib=lib)
    b, _ = oracle.proj(mu.codes, mu.scales, g, x, lib=lib)
    ref = (torch.nn.functional.silu(torch.from_numpy(a)) * torch.from_numpy(b)).numpy()
    assert np.allclose(h, ref, rtol=1e-13, atol=1e-300)
    cols = np.array([0, 7, 8, 15, 16, 47])
    hc, _ = oracle.silu_mul_cols(codes, scales, g, x, F, cols=cols, lib=lib)
    assert np.array_equal(hc, h[:, cols])


def pin_silu_mul_bound(lib):
    """The allowance: max |silu'| over a fine grid stays below the 1.1 the
    bound uses; a bound-sized perturbation of gate and up moves h by no more
    than the bound; and the bf16 acceptance test passes a correctly rounded
    value and fails one an allowance away."""
    z = torch.linspace(-40.0, 40.0, 800001, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(z).sum().backward()
    assert z.grad.abs().max().item() < 1.1
    rng = np.random.default_rng(6)
    a = rng.normal(0, 4, 2000)
    b = rng.normal(0, 4, 2000)
    Sa = np.abs(a) * rng.uniform(1, 50, a.size)
    Sb = np.abs(b) * rng.uniform(1, 50, b.size)
    bound = np.empty(a.size)
    lib.orc_silu_mul_bound(a.size, a.ctypes.data, b.ctypes.data, Sa.ctypes.data, Sb.ctypes.data,
                           oracle.RTOL, bound.ctypes.data)
    for sa in (-1, 1):
        for sb in (-1, 1):
            a2 = a + sa * oracle.RTOL * Sa
            b2 = b + sb * oracle.RTOL * Sb
            moved = np.abs(oracle.silu_mul(a2, b2, lib) - oracle.silu_mul(a, b, lib))
            assert (moved <= bound * (1 + 1e-12)).all()
    href = np.array([1.0, -3.0, 0.0, np.nan, 100.0])
    bd = np.array([0.0, 0.01, 0.0, 0.0, 0.5])
    ok = torch.tensor([1.0, -3.0078125, 0.0, float("nan"), 100.5], dtype=torch.bfloat16)
    bits = ok.view(torch.int16).numpy().view(np.uint16)
    bad, _ = oracle.check_bf16(href, bd, bits, lib)
    assert bad == 0, bad
    for i, v in [(0, 1.0078125 * 1.0078125), (2, 1e-30), (3, 1.0), (4, 102.0)]:
        t = ok.clone()
        t[i] = v
        bad, _ = oracle.check_bf16(href, bd, t.view(torch.int16).numpy().view(np.uint16), lib)
        assert bad == 1, (i, v, bad)


# ---- greedy argmax acceptance ----------------------------------------------

def pin_argmax_check(lib):
    """The argmax acceptance test: with a clear maximum only torch.argmax's
    index (and a value within tolerance of it) passes; two logits within
    tolerance of each other both pass, one clearly below does not; a row
    with NaNs accepts only its first NaN column with a NaN value; indices out
    of range fail."""
    rng = np.random.default_rng(13)
    M, N = 3, 50
    y = rng.normal(0, 1, (M, N))
    S = np.full((M, N), 1.0)
    rt = 1e-3                                        # tolerance 1e-3 per element
    y[0, 17] = 10.0                                  # clear maximum
    y[1, 3], y[1, 40] = 5.0, 5.0015                  # within 2e-3 of each other
    y[1, 41] = 4.99                                  # clearly below
    y[2, 9] = np.nan
    y[2, 30] = np.nan
    want0 = int(torch.argmax(torch.from_numpy(y[0])))
    assert want0 == 17

    def run(rows_idx, rows_val):
        return oracle.argmax_check(y, S, np.array(rows_idx), np.array(rows_val, np.float32),
                                   rtol=rt, lib=lib)

    base_i, base_v = [17, 40, 9], [10.0, 5.0015, np.nan]
    assert run(base_i, base_v) == 0
    assert run([3, 3, 9], [10.0, 5.0, np.nan]) == 1          # row 0: not the maximum
    assert run([17, 3, 9], [10.0, 5.0, np.nan]) == 0         # row 1: within tolerance
    assert run([17, 41, 9], [10.0, 4.99, np.nan]) == 1       # row 1: clearly below
    assert run([17, 40, 30], [10.0, 5.0015, np.nan]) == 1    # row 2: not the first NaN
    assert run([17, 40, 9], [10.0, 5.0015, 1.0]) == 1        # row 2: value not NaN
    assert run([17, 40, 9], [10.002, 5.0015, np.nan]) == 1   # row 0: value off
    assert run([-1, 40, 9], [10.0, 5.0015, np.nan]) == 1
    assert run([17, N, 9], [10.0, 5.0015, np.nan]) == 1


# ---- the NVFP4 quantizer ----------------------------------------------------

def golden_e2m1_rounding():
    rows = []
    for line in open(os.path.join(GOLDEN, "e2m1_rne_ocp_mx_v1.txt")):
        if line.strip() and not line.startswith("#"):
            v, c = line.split()
            rows.append((float(v), int(c, 16)))
    return rows


def pin_quant_e2m1_rounding(lib):
    """e2m1 rounding against the OCP MX conversion rule, tabulated: the code of
    |w| = v under scale 1.0 (0x38) and g = 1, and the same under scale 0.5
    (0x30) and g = 2^-7 for |w| = v * 2^-8 (exact); saturation past 6."""
    rows = golden_e2m1_rounding()
    assert len(rows) >= 20
    for v, c in rows:
        assert lib.orc_quant_code(v, 0x38, 1.0) == c, (v, c, lib.orc_quant_code(v, 0x38, 1.0))
        if v < 1e29:
            assert np.float32(v * 2.0 ** -8) * np.float32(2.0 ** 8) == np.float32(v)
            assert lib.orc_quant_code(v * 2.0 ** -8, 0x30, 2.0 ** -7) == c, v
    assert lib.orc_quant_code(float("inf"), 0x38, 1.0) == 7
    assert lib.orc_quant_code(1.0, 0x00, 1.0) == 0            # scale 0: code 0


def _f32_22(v):
    """v rounded to 22 significant bits (so that 0.375 v stays exact in fp32)"""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.round(m * 2.0 ** 22) / 2.0 ** 22, e).astype(np.float32)


def pin_quant_e4m3_torch(lib):
    """e4m3 scale rounding against torch's float8_e4m3fn cast (round to nearest
    even) of t = amax_b / (6 g), with g a power of two so that amax_b = 6 g t
    is exact: every value, every midpoint between neighbours, the 22-bit
    neighbours of every midpoint, random values in [0, 448] and below 2^-6;
    saturation above 448 in closed form."""
    vals = pins_e4m3_positive()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1].astype(np.float64) + vals[1:]) / 2)
    rng = np.random.default_rng(9)
    up = _f32_22(mids.astype(np.float64) * (1 + 2.0 ** -21))
    dn = _f32_22(mids.astype(np.float64) * (1 - 2.0 ** -21))
    assert (up > mids).all() and (dn < mids).all()
    t = np.concatenate([vals, mids, up, dn, _f32_22(rng.uniform(0, 448, 3000)),
                        _f32_22(2.0 ** rng.uniform(-12, -5, 1000))])
    want = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for g in (2.0 ** -4, 2.0 ** -20, 2.0 ** 3):
        a = t.astype(np.float64) * 6.0 * g
        assert np.array_equal(a.astype(np.float32).astype(np.float64), a)
        got = np.array([lib.orc_quant_scale(float(v), g) for v in a])
        assert np.array_equal(got, want), (g, t[got != want][:5])
    for v in (448.0001, 460.0, 464.0, 1e6, float("inf")):
        assert lib.orc_quant_scale(v * 6 * 2.0 ** -4, 2.0 ** -4) == 0x7E


def pins_e4m3_positive():
    """The 127 non-negative finite e4m3 values in code order (torch's decoder)."""
    return torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


# exact rational reference of the quantiser's two rounding steps: the grid
# value nearest to a rational quotient, ties to the even code, found with
# fractions.Fraction (every float is an exact rational)

def _fr_grids():
    e4 = [Fraction(float(v)) for v in pins_e4m3_positive()]
    table = golden_e2m1()
    e2 = [Fraction(table[c]) for c in range(8)]
    return e4, e2


def _fr_nearest(q, grid):
    i = bisect.bisect_left(grid, q)
    if i == 0:
        return 0
    if i == len(grid):
        return len(grid) - 1
    dl, du = q - grid[i - 1], grid[i] - q
    if dl < du:
        return i - 1
    if du < dl:
        return i
    return i - 1 if (i - 1) % 2 == 0 else i


def fr_quant_scale(a, g, e4):
    return _fr_nearest(Fraction(a) / (6 * Fraction(g)), e4)


def fr_quant_code(a, s, g, e4, e2):
    if s == 0:
        return 0
    return _fr_nearest(Fraction(a) / (e4[s] * Fraction(g)), e2)


def fr_quantize(bits, N, K):
    """The quantiser's definition in exact rationals: g = fp32(amax / 2688)
    (numpy's IEEE fp32 division), then per block the nearest e4m3 scale and per
    element the nearest e2m1 magnitude with w's sign bit."""
    e4, e2 = _fr_grids()
    wv = pins_bf16_of(np.ascontiguousarray(bits, np.uint16).ravel()).reshape(N, K)
    amax = np.abs(wv).max()
    g = 1.0 if amax == 0 else float(np.float32(amax) / np.float32(2688.0))
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    sign = (np.ascontiguousarray(bits, np.uint16).reshape(N, K) >> 15).astype(np.uint8)
    for n in range(N):
        for b in range(K // 16):
            blk = np.abs(wv[n, 16 * b:16 * b + 16])
            s = fr_quant_scale(float(blk.max()), g, e4)
            scales[n, b] = s
            q = [fr_quant_code(float(a), s, g, e4, e2) | (int(sign[n, 16 * b + i]) << 3 if s else 0)
                 for i, a in enumerate(blk)]
            codes[n, 8 * b:8 * b + 8] = [q[2 * i] | (q[2 * i + 1] << 4) for i in range(8)]
    return codes, scales, g


def pin_quant_fraction(lib):
    """orc_quant_scale / orc_quant_code against the exact rational reference on
    random values under random fp32 global scales (normal, subnormal and
    large), and on quotients constructed within one fp32 step of every
    midpoint: a = bf16 w with g = fp32(w / (mid * v)) and its fp32 neighbours,
    where fp32 evaluations of the quotient decide wrongly."""
    e4, e2 = _fr_grids()
    rng = np.random.default_rng(13)
    gs = np.concatenate([np.float32(2.0 ** rng.uniform(-30, -5, 24)),
                         np.float32(2.0 ** rng.uniform(-148, -127, 4)),
                         np.float32(2.0 ** rng.uniform(5, 30, 4))]).astype(np.float64)
    for g in gs:
        a = (np.abs(rng.normal(0, 1, 40)) * 2688 * g / 3).astype(np.float32).astype(np.float64)
        for v in a:
            assert lib.orc_quant_scale(v, g) == fr_quant_scale(v, g, e4), (v, g)
            s = int(rng.integers(0, 0x7F))
            assert lib.orc_quant_code(v, s, g) == fr_quant_code(v, s, g, e4, e2), (v, s, g)
    w = pins_bf16_of(rng.integers(0x3C00, 0x3F00, 120).astype(np.uint16))    # bf16 in [2^-7, 0.5)
    mids_e2 = [(e2[i] + e2[i + 1]) / 2 for i in range(7)]
    mids_e4 = [(e4[i] + e4[i + 1]) / 2 for i in range(0x7E)]
    near = 0
    for k, v in enumerate(w):
        s = int(rng.integers(1, 0x7F))
        mu = mids_e2[k % 7]
        g0 = np.float32(v / float(mu * e4[s]))
        for g in (np.nextafter(g0, np.float32(0)), g0, np.nextafter(g0, np.float32(1))):
            g = float(g)
            want = fr_quant_code(v, s, g, e4, e2)
            assert lib.orc_quant_code(v, s, g) == want, (v, s, g)
            # the quotient evaluated in fp32 (1 / (s g), then times |w|) on the
            # other side of the midpoint than the exact one
            exact = Fraction(v) / (e4[s] * Fraction(g))
            r32 = Fraction(float(np.float32(v) * (np.float32(1) / (np.float32(float(e4[s]))
                                                                   * np.float32(g)))))
            near += int((r32 > mu) != (exact > mu) or (r32 == mu) != (exact == mu))
        m = mids_e4[(7 * k) % 0x7E]
        g0 = np.float32(v / float(6 * m))
        for g in (np.nextafter(g0, np.float32(0)), g0, np.nextafter(g0, np.float32(1))):
            g = float(g)
            assert lib.orc_quant_scale(v, g) == fr_quant_scale(v, g, e4), (v, g)
    assert near > 0          # the construction does reach quotients fp32 misplaces


def pin_quantize_fraction(lib):
    """orc_quantize against the exact rational definition (fr_quantize) on the
    tensors built at and next to the rounding ties (tests/quant_inputs.py):
    g = 2^-7 with exact ties (ties to the even code), and a g of 24
    significant bits with hundreds of elements within 2^-23 of a tie."""
    import quant_inputs
    for kind in ("pow2", "near"):
        bits, _ = quant_inputs.tie_weights(kind, K=256)
        N, K = bits.shape
        codes, scales, g = oracle.quantize(bits, N, K, lib=lib)
        rc, rs, rg = fr_quantize(bits, N, K)
        assert g == rg, (kind, g, rg)
        assert np.array_equal(scales, rs), (kind, np.argwhere(scales != rs)[:5])
        assert np.array_equal(codes, rc), (kind, np.argwhere(codes != rc)[:5])


def pin_quant_global_scale(lib):
    """g = amax / 2688 as one fp32 division (numpy's IEEE float32), 1 for an
    all-zero tensor (also of negative zeros)."""
    rng = np.random.default_rng(10)
    for scale in (0.02, 3e-39, 1e30):
        w = torch.from_numpy(rng.normal(0, 1, 4096) * scale).to(torch.bfloat16)
        bits = w.view(torch.int16).numpy().view(np.uint16)
        amax = np.float32(np.abs(w.float().numpy()).max())
        assert oracle.quant_global_scale(bits, lib) == np.float32(amax) / np.float32(2688)
    assert oracle.quant_global_scale(np.zeros(64, np.uint16), lib) == 1.0
    assert oracle.quant_global_scale(np.full(64, 0x8000, np.uint16), lib) == 1.0


def pin_quantize_exact_recovery(lib):
    """Weights that are exactly q * s * g, every block holding a +-6 element
    and one block the scale 448 (so the tensor's amax is 2688 g), come back
    as the same codes and scales."""
    rng = np.random.default_rng(11)
    N, K = 12, 256
    g = 2.0 ** -14
    e4 = pins_e4m3_positive()
    e2 = np.array([lib.orc_e2m1(c) for c in range(16)])
    s = rng.integers(0x08, 0x7F, (N, K // 16)).astype(np.uint8)      # normal scales
    s[3, 5] = 0x7E
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    q[:, ::16] = rng.choice([7, 15], (N, K // 16))                      # one +-6 per block
    w = e2[q] * np.repeat(e4[s].astype(np.float64), 16, axis=1) * g
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pins_bf16_of(bits), w)                        # exact in bf16
    codes, scales, gq = oracle.quantize(bits, N, K, lib=lib)
    assert gq == g
    assert np.array_equal(scales, s)
    assert np.array_equal(codes, (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8))


def pins_bf16_of(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def pin_quantize_nearest(lib):
    """orc_quantize against the exact rational definition on random N(0, 0.02)
    weights with zero blocks, blocks small enough for subnormal and zero
    e4m3 scales, negative zeros and one large element setting g: every
    scale and code exactly, zero blocks giving scale 0 and codes 0."""
    rng = np.random.default_rng(12)
    N, K = 24, 512
    w = rng.normal(0, 0.02, (N, K))
    w[2] = 0.0
    w[3, :64] = 0.0
    w[4, :256] *= 1e-4                             # subnormal e4m3 scales
    w[4, 256:] *= 1e-6                             # zero e4m3 scales
    w[5, 7] = 0.9                                  # the tensor's amax
    w[6, ::3] = -0.0
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, g = oracle.quantize(bits, N, K, lib=lib)
    rc, rs, rg = fr_quantize(bits, N, K)
    assert g == rg
    assert np.array_equal(scales, rs), np.argwhere(scales != rs)[:5]
    assert np.array_equal(codes, rc), np.argwhere(codes != rc)[:5]
    assert (scales[2] == 0).all() and (scales[3, :4] == 0).all()
    assert (scales[4] < 0x08).any() and (scales[4] == 0).any()
    assert (codes[2] == 0).all()


ALL_PINS = [pin_e2m1_table, pin_e4m3_torch, pin_e4m3_landmarks, pin_bf16_torch,
            pin_dequant_rows, pin_exact_tiny_fast, pin_abs_sum, pin_one_hot,
            pin_invariants, pin_nan_scale, pin_check, pin_silu_mul_torch,
            pin_silu_mul_fused_rows, pin_silu_mul_bound, pin_quant_e2m1_rounding,
            pin_quant_e4m3_torch, pin_quant_global_scale, pin_quantize_exact_recovery,
            pin_argmax_check, pin_quant_fraction, pin_quantize_nearest,
            pin_quantize_fraction]
