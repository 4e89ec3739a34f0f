"""q4proj_quantize (bf16 -> NVFP4 codes, e4m3 block scales, global scale)
against the CPU oracle, bit for bit.  Every rounding decision is the nearest
value to an exact quotient (ties to the even code); the oracle takes it in
exact fp64 comparisons (pinned to exact rationals), the kernel by an fp32
estimate bracketed and corrected with exact fma comparisons.

* random N(0, 0.02) weights on small and ragged shapes (every element);
* special tensors: all zero, negative zeros, zero and tiny blocks, bf16
  subnormals and extremes, exact e2m1 and e4m3 rounding ties;
* every element and scale tie of every scale code, exactly on the tie
  (g = 2^-7) and within 2^-23 of it (a g of 24 significant bits), one bf16
  step either side, in blocks of their own;
* the fused gate/up shape (34816 x 5120) on sampled rows, g over the whole
  tensor;
* quantize -> pack -> gemv on the GPU against the oracle projection of the
  oracle's own quantization; repeatability.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_inputs
import synth
from gpu_util import DEV, assert_parity, note, pack, project, q4

pytestmark = pytest.mark.gpu


def run_quant(bits, N, K):
    w = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV)
    codes, scales, g = q4().quantize_weight(w.reshape(-1), N, K)
    torch.cuda.synchronize()
    return (codes.cpu().numpy().reshape(N, K // 2), scales.cpu().numpy().reshape(N, K // 16),
            float(g.item()))


def assert_same(bits, N, K, rows=None):
    note(f"quantize N={N} K={K}")
    c, s, g = run_quant(bits, N, K)
    rc, rs, rg = oracle.quantize(bits, N, K, rows=rows)
    assert np.float32(g) == np.float32(rg), (g, rg)
    if rows is not None:
        c, s = c[rows], s[rows]
    bad_s = np.argwhere(s != rs)
    assert bad_s.size == 0, (bad_s[:5], s[tuple(bad_s[0])], rs[tuple(bad_s[0])])
    bad_c = np.argwhere(c != rc)
    assert bad_c.size == 0, (bad_c[:5], c[tuple(bad_c[0])], rc[tuple(bad_c[0])])
    return c, s, g


def normal_bits(seed, N, K, std=0.02):
    return synth.normal_bf16(seed, 400, N * K, std=std).reshape(N, K)


SHAPES = [(1, 16), (3, 48), (17, 256), (64, 1040), (300, 5120), (5, 16000), (1, 2 ** 20)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_random_shapes(N, K):
    assert_same(normal_bits(N + K, N, K), N, K)


def bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_zero_tensors():
    for fill in (0x0000, 0x8000):
        bits = np.full((4, 64), fill, np.uint16)
        c, s, g = assert_same(bits, 4, 64)
        assert g == 1.0 and not c.any() and not s.any()


def test_zero_tiny_and_extreme_blocks():
    rng = np.random.default_rng(20)
    N, K = 16, 512
    w = rng.normal(0, 0.02, (N, K))
    w[1] = 0.0
    w[2, :128] = -0.0
    w[3, :256] *= 1e-4                      # subnormal e4m3 scales
    w[3, 256:] *= 1e-6                      # zero e4m3 scales
    w[4, 5] = 0.9
    w[5, ::2] *= -1
    bits = bf16_bits(w)
    bits[6, :16] = 0x0001                   # smallest bf16 subnormal
    bits[6, 16:32] = 0x8001
    bits[7, 0] = 0x7F7F                     # largest bf16
    bits[7, 1] = 0xFF7F
    assert_same(bits, N, K)
    # a tensor of bf16 subnormals only: g itself is an fp32 subnormal
    tiny = (np.random.default_rng(21).integers(0, 128, (4, 64)) |
            (np.random.default_rng(22).integers(0, 2, (4, 64)) << 15)).astype(np.uint16)
    assert_same(tiny, 4, 64)
    huge = bf16_bits(np.random.default_rng(23).normal(0, 1e37, (4, 64)))
    assert_same(huge, 4, 64)


def test_rounding_ties():
    """Exact e2m1 midpoints (|w| / unit = 0.25, 0.75, ..., 5) with power-of-two
    scales, and blocks whose (amax_b / 6) / g lands on e4m3 midpoints."""
    g = 2.0 ** -14
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for e in range(-6, 9):                       # scale 2^e (e4m3 normal, mantissa 0)
        s = 2.0 ** e
        blk = np.concatenate([[6.0], mids, -mids, [0.5]])[:16] * s * g
        rows.append(blk)
    # t on e4m3 midpoints: amax_b / 6 / g = (v_c + v_c+1) / 2 for codes 0x30..0x3F
    e4 = torch.arange(0x30, 0x41, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(16):
        t = (e4[c] + e4[c + 1]) / 2
        rows.append(np.full(16, t * 6 * g) * np.where(np.arange(16) % 2, -1, 1))
    rows.append(np.full(16, 448 * 6 * g))        # the tensor's amax: g is exact
    w = np.array(rows)
    bits = bf16_bits(w)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
                          .numpy(), w)
    N = w.shape[0]
    c, s, gq = assert_same(bits, N, 16)
    assert gq == g


@pytest.mark.parametrize("kind", ["pow2", "near"])
def test_tie_tensors(kind):
    bits, amax = quant_inputs.tie_weights(kind)
    N, K = bits.shape
    c, s, g = assert_same(bits, N, K)
    assert g == np.float32(amax) / np.float32(2688)


def test_fused_gate_up_shape_sampled_rows():
    N, K = 34816, 5120
    bits = normal_bits(7, N, K)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, N - 1],
                                     np.random.default_rng(24).choice(N, 59, replace=False)]))
    assert_same(bits, N, K, rows=rows)


def test_quantize_pack_project():
    N, K, M = 1040, 2064, 3
    bits = normal_bits(30, N, K)
    note(f"quantize -> pack -> gemv N={N} K={K}")
    w = torch.from_numpy(bits.view(np.int16)).to(DEV).reshape(-1)
    codes, scales, g = q4().quantize_weight(w, N, K)
    packed = q4().pack_weight(codes, scales, N, K)
    x = synth.x_bf16(30, 1, M, K)
    gval = float(g.item())
    y = project("gemv", packed, gval, x, N, K)
    rc, rs, rg = oracle.quantize(bits, N, K)
    assert np.float32(rg) == np.float32(gval)
    assert_parity(rc, rs, rg, x, y)


def test_repeatable():
    N, K = 333, 4096
    bits = normal_bits(31, N, K)
    a = run_quant(bits, N, K)
    b = run_quant(bits, N, K)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
