"""Bounded soak of the stream-K exchange and the argmax protocol: about three
thousand launches back to back, no synchronisation between them, over shapes
whose tiles are shared between workgroups (exchange words), whose K is split
into joined ranges, with the fused silu epilogue and with the greedy argmax
(including exact ties between distant columns).  Every call uses the same
caller-owned workspace, so each must leave it zero-filled for the next.

Each case's result of one eager launch (launch, synchronise) is its
reference; every soak launch writes its own output slot and is compared bit
for bit with it, stopping at the first mismatch.  The argmax references are
also checked against the oracle, and where the logits are written, against
them: the index is the first column holding the row's largest logit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_parity, note, pack, q4, to_dev_x

pytestmark = pytest.mark.gpu

SLOTS = 8                 # outputs per case per round
TARGET_LAUNCHES = 3000


class Case:
    def __init__(self, name, launch, outputs):
        self.name, self.launch, self.outputs = name, launch, outputs   # launch(slot)
        self.ref = None


def _matrix(seed, N, K):
    return synth.nvfp4_normal_matrix(seed, 1, N, K, threads=8)


def test_soak_back_to_back_bitwise():
    m = q4()
    cases, needs = [], [0]

    def gemv_case(seed, M, N, K):
        mat = _matrix(seed, N, K)
        pc, ps = pack(mat.codes, mat.scales, N, K)
        x = synth.x_bf16(seed, 2, M, K, threads=1)
        xd = to_dev_x(x)
        ys = [torch.empty((M, N), dtype=torch.float32, device=DEV) for _ in range(SLOTS + 1)]
        needs.append(m.q4proj_workspace_bytes(M, N, K))
        c = Case(f"gemv M={M} N={N} K={K}",
                 lambda s: m.q4proj_gemv(pc, ps, mat.g, xd, ys[s], M, N, K, workspace=ws[0]),
                 lambda s: [ys[s]])
        c.check = lambda: assert_parity(mat.codes, mat.scales, mat.g, x, ys[SLOTS].cpu().numpy(),
                                        rows=np.arange(0, N, max(1, N // 512)))
        return c

    def silu_case(seed, M, F, K):
        mat = _matrix(seed, 2 * F, K)
        pc, ps = pack(mat.codes, mat.scales, 2 * F, K)
        xd = to_dev_x(synth.x_bf16(seed, 2, M, K, threads=1))
        hs = [torch.empty((M, F), dtype=torch.int16, device=DEV) for _ in range(SLOTS + 1)]
        needs.append(m.q4proj_silu_mul_workspace_bytes(M, F, K))
        c = Case(f"gemv_silu_mul M={M} F={F} K={K}",
                 lambda s: m.q4proj_gemv_silu_mul(pc, ps, mat.g, xd, hs[s], M, F, K,
                                                  workspace=ws[0]),
                 lambda s: [hs[s]])
        c.check = lambda: None
        return c

    def argmax_case(seed, M, N, K, with_logits):
        half = _matrix(seed, N // 2, K)
        # rows j and j + N/2 are the same weight row: every logit appears
        # twice (equal up to the order the two tiles are summed in), so the
        # maximum is a tie or a near-tie between distant columns
        codes = np.concatenate([half.codes, half.codes])
        scales = np.concatenate([half.scales, half.scales])
        pc, ps = pack(codes, scales, N, K)
        x = synth.x_bf16(seed, 3, M, K, threads=1)
        xd = to_dev_x(x)
        vals = [torch.empty(M, dtype=torch.float32, device=DEV) for _ in range(SLOTS + 1)]
        idxs = [torch.empty(M, dtype=torch.int64, device=DEV) for _ in range(SLOTS + 1)]
        ys = [torch.empty((M, N), dtype=torch.float32, device=DEV) if with_logits else None
              for _ in range(SLOTS + 1)]
        needs.append(m.q4proj_argmax_workspace_bytes(M, N, K))
        c = Case(f"gemv_argmax M={M} N={N} K={K} logits={with_logits}",
                 lambda s: m.q4proj_gemv_argmax(pc, ps, half.g, xd, ys[s], vals[s], idxs[s], M,
                                                N, K, workspace=ws[0]),
                 lambda s: [vals[s], idxs[s]] + ([ys[s]] if with_logits else []))

        def check():
            yr, S = oracle.proj(codes, scales, half.g, x)
            idx = idxs[SLOTS].cpu().numpy()
            val = vals[SLOTS].cpu().numpy()
            assert oracle.argmax_check(yr, S, idx, val) == 0
            if with_logits:
                # against its own logits: the first column holding the row's
                # largest value, and that value bit for bit
                y = ys[SLOTS].cpu().numpy()
                first = np.argmax(y, axis=1)
                assert np.array_equal(idx, first), (idx, first)
                assert np.array_equal(val.view(np.uint32),
                                      y[np.arange(M), first].view(np.uint32))
        c.check = check
        return c

    ws = [None]
    note("soak: building cases")
    cases = [gemv_case(60, 1, 17408, 5120), gemv_case(61, 1, 5120, 17408),
             gemv_case(62, 7, 5120, 17408), gemv_case(63, 16, 17408, 5120),
             gemv_case(64, 13, 300, 1040), silu_case(65, 2, 4096, 2560),
             argmax_case(66, 1, 65536, 5120, False), argmax_case(67, 7, 65536, 5120, True)]
    ws[0] = torch.zeros(max(needs), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()

    # eager references: one launch each, synchronised, checked against the oracle
    for c in cases:
        note(f"soak reference: {c.name}")
        c.launch(SLOTS)
        torch.cuda.synchronize()
        c.ref = [t.clone() for t in c.outputs(SLOTS)]
        c.check()
    assert int(ws[0].count_nonzero()) == 0, "workspace not left zero-filled"

    def same(a, b):
        if a.dtype == torch.float32:
            return torch.equal(a.view(torch.int32), b.view(torch.int32))
        return torch.equal(a, b)

    launches, rnd = 0, 0
    while launches < TARGET_LAUNCHES:
        note(f"soak round {rnd}: {launches} launches so far")
        for s in range(SLOTS):
            for c in cases:
                c.launch(s)
        launches += SLOTS * len(cases)
        torch.cuda.synchronize()
        for c in cases:
            for s in range(SLOTS):
                for k, (got, want) in enumerate(zip(c.outputs(s), c.ref)):
                    assert same(got, want), (f"round {rnd}, {c.name}, slot {s}, output {k}: "
                                             f"differs from the eager result")
        assert int(ws[0].count_nonzero()) == 0, f"round {rnd}: workspace left dirty"
        rnd += 1
    note(f"soak: {launches} launches, all bit-identical to the eager results")
