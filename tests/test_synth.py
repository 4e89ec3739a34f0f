"""The seeded input generator: determinism, encoders, workload statistics."""
import math

import numpy as np
import pytest
import torch

import pins
import synth


def test_counter_based_and_thread_invariant():
    a = synth.normal_bf16(3, 7, 10001, threads=1)
    b = synth.normal_bf16(3, 7, 10001, threads=8)
    assert np.array_equal(a, b)
    lib = synth.load()
    single = np.zeros(1, np.uint16)
    lib.syn_normal_bf16(3, 7, 1.0, 5000, 1, single.ctypes.data)
    assert single[0] == a[5000]
    m1 = synth.nvfp4_normal_matrix(5, 1, 33, 96, threads=1)
    m2 = synth.nvfp4_normal_matrix(5, 1, 33, 96, threads=7)
    assert np.array_equal(m1.codes, m2.codes) and np.array_equal(m1.scales, m2.scales)
    assert m1.g == m2.g


def test_streams_differ():
    assert not np.array_equal(synth.normal_bf16(1, 100, 64), synth.normal_bf16(1, 101, 64))
    assert not np.array_equal(synth.normal_bf16(1, 100, 64), synth.normal_bf16(2, 100, 64))


def test_normal_statistics():
    x = pins.torch_bf16(synth.normal_bf16(9, 1, 200000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 0.005


def test_bf16_encoder_matches_torch_rne():
    lib = synth.load()
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                           [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([lib.syn_encode_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_e4m3_encoder_matches_torch_rne():
    lib = synth.load()
    rng = np.random.default_rng(1)
    vals = np.concatenate([np.abs(rng.standard_normal(4000)) * 2.0 ** rng.integers(-12, 9, 4000),
                           pins.torch_e4m3_table()[:0x7F]])
    vals = vals[vals < 448.0]
    # midpoints between consecutive codes exercise ties-to-even
    tab = pins.torch_e4m3_table()[:0x7F]
    vals = np.concatenate([vals, (tab[:-1] + tab[1:]) / 2])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([lib.syn_encode_e4m3(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref), vals[got != ref][:5]
    assert lib.syn_encode_e4m3(1000.0) == 0x7E


def test_e2m1_encoder_nearest_ties_even():
    lib = synth.load()
    table = pins.golden_e2m1()
    mags = [table[c] for c in range(8)]
    rng = np.random.default_rng(2)
    vals = list(rng.uniform(-7, 7, 3000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 9.0]
    for v in vals:
        code = lib.syn_encode_e2m1(float(v))
        a = min(abs(v), 6.0)
        dists = [abs(a - m) for m in mags]
        best = min(dists)
        cands = [c for c in range(8) if dists[c] == best]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert code & 7 == want, (v, code)
        assert (code >> 3) == (1 if math.copysign(1, v) < 0 else 0)


def test_tiny_workload_statistics():
    (case,) = synth.workload_cases("tiny", cache=False)
    assert (case.M, case.N, case.K) == (1, 512, 256)
    codes = np.concatenate([case.matrix.codes & 15, case.matrix.codes >> 4]).ravel()
    hist = np.bincount(codes, minlength=16) / codes.size
    assert hist.min() > 0.05 and hist.max() < 0.075          # uniform over 16
    s = pins.torch_e4m3_table()[case.matrix.scales.ravel()]
    assert s.min() >= 0.009 and s.max() < 3.5
    assert (case.matrix.scales < 8).mean() > 0.0             # some subnormal scales
    assert case.matrix.g == 1.0


def test_normal_weight_quantiser_statistics():
    m = synth.nvfp4_normal_matrix(1, synth.STREAM_W, 256, 5120)
    codes = np.concatenate([m.codes & 15, m.codes >> 4]).ravel()
    hist = np.bincount(codes, minlength=16) / codes.size
    assert (hist > 0.02).all()                                # every code used
    assert abs(hist[7] - hist[15]) < 0.005                    # symmetric
    assert 3e-5 < m.g < 6e-5                                  # amax ~ 0.1 / 2688
    s = pins.torch_e4m3_table()[m.scales.ravel()]
    assert (s >= 2 ** -6).all() and s.max() <= 448.0          # normal scales only


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_shapes(name):
    seed, M, mats = synth.WORKLOADS[name]
    assert seed == synth.WORKLOAD_ORDER.index(name)
    for _, _, _, N, K in mats:
        assert K % 256 == 0 and N % 256 == 0
