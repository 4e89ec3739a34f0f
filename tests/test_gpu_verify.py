"""The verify GEMV at its full sizes: every M from 1 to 16 on both MLP
matrices of the 27B-style model (gate/up 5120 -> 17408, down 17408 -> 5120),
the shapes bench.py's verify sweep times, against the oracle on sampled
output columns (every 32nd and the last 16) for every activation row.

At these sizes the launcher runs gate/up with one K range up to M = 14 and
two above, and down with one range at M = 1, two at M = 2-4 and four at
M = 5-16; above M = 4 the exchanges carry two rows per word.
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_parity, note, pack, project

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mat", ["gate_up", "down"])
def test_verify_full_size_every_m(mat):
    (case,) = synth.workload_cases("mtp", only=[mat])
    w = case.matrix
    N, K = w.N, w.K
    packed = pack(w.codes, w.scales, N, K)
    cols = np.unique(np.concatenate([np.arange(0, N, 32), np.arange(N - 16, N)]))
    for M in range(1, 17):
        x = synth.x_bf16(70 + M, 5, M, K)
        note(f"verify gemv {mat} M={M} N={N} K={K}")
        y = project("gemv", packed, w.g, x, N, K)
        assert_parity(w.codes, w.scales, w.g, x, y, rows=cols)
