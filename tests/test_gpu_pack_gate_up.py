"""q4proj_pack_gate_up: the fused gate/up weight built from a checkpoint's two
separate NVFP4 weights.

* the packed bytes equal q4proj_pack of the [2F][K] weight whose rows
  alternate 8 gate rows and 8 up rows (the row order of the fused layout),
  on ragged and full MLP shapes;
* q4proj_gemv_silu_mul and q4proj_gemm_silu_mul on that pack against the
  oracle's silu(gate) * up computed from the two separate weights (no row
  interleave in the reference);
* unequal global scales are refused.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, note, q4, to_dev_u8, to_dev_x

pytestmark = pytest.mark.gpu


def split_gate_up(fused, F):
    """rows of a [2F][...] array in the fused order -> (gate, up), each [F][...]"""
    blk = fused.reshape(F // 8, 2, 8, -1)
    return (np.ascontiguousarray(blk[:, 0].reshape(F, -1)),
            np.ascontiguousarray(blk[:, 1].reshape(F, -1)))


def packed_pair(F, K, seed):
    fm = synth.nvfp4_normal_matrix(seed, 1, 2 * F, K, threads=8)
    gc, uc = split_gate_up(fm.codes, F)
    gs, us = split_gate_up(fm.scales, F)
    m = q4()
    note(f"pack_gate_up F={F} K={K}")
    pc, ps = m.pack_gate_up_weight(to_dev_u8(gc).reshape(-1), to_dev_u8(gs).reshape(-1),
                                   to_dev_u8(uc).reshape(-1), to_dev_u8(us).reshape(-1),
                                   fm.g, fm.g, F, K)
    rc, rs = m.pack_weight(to_dev_u8(fm.codes).reshape(-1), to_dev_u8(fm.scales).reshape(-1),
                           2 * F, K)
    torch.cuda.synchronize()
    return fm, (gc, gs, uc, us), (pc, ps), (rc, rs)


@pytest.mark.parametrize("F,K", [(8, 16), (24, 208), (1040, 1040), (17408, 5120)])
def test_same_bytes_as_packing_the_fused_rows(F, K):
    _, _, (pc, ps), (rc, rs) = packed_pair(F, K, 60 + F % 97)
    assert torch.equal(pc, rc) and torch.equal(ps, rs)


@pytest.mark.parametrize("M", [1, 7, 40])
def test_silu_mul_on_the_pack_against_separate_weights(M):
    F, K = 1024, 2064
    fm, (gc, gs, uc, us), (pc, ps), _ = packed_pair(F, K, 61)
    x = synth.x_bf16(61, 2 + M, M, K, threads=1)
    h_ref, bound = oracle.silu_mul_separate(gc, gs, uc, us, fm.g, x)
    m = q4()
    fns = [m.q4proj_gemm_silu_mul] + ([m.q4proj_gemv_silu_mul] if M <= 16 else [])
    for fn in fns:
        h = torch.empty((M, F), dtype=torch.int16, device=DEV)
        note(f"{fn.__name__} on the gate/up pack M={M} F={F} K={K}")
        fn(pc, ps, fm.g, to_dev_x(x), h, M, F, K)
        torch.cuda.synchronize()
        bad, worst = oracle.check_bf16(h_ref, bound, h.cpu().numpy().view(np.uint16))
        assert bad == 0, (fn.__name__, bad, worst)


def test_unequal_global_scales_refused():
    m = q4()
    F, K = 16, 128
    z = torch.zeros(F * K // 2, dtype=torch.uint8, device=DEV)
    s = torch.zeros(F * K // 16, dtype=torch.uint8, device=DEV)
    pc = torch.empty(m.q4proj_packed_codes_bytes(2 * F, K), dtype=torch.uint8, device=DEV)
    ps = torch.empty(m.q4proj_packed_scales_bytes(2 * F, K), dtype=torch.uint8, device=DEV)
    with pytest.raises(m.Q4ProjError) as e:
        m.q4proj_pack_gate_up(z, s, z.clone(), s.clone(), 0.5, 0.25, F, K, pc, ps)
    assert e.value.status == m.EINVAL
