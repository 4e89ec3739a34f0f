"""q4proj_pack / q4proj_unpack on the GPU: the documented tile layout, exact
round trip, zero padding and determinism (byte work: bit-exact)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, note, q4, to_dev_u8

pytestmark = pytest.mark.gpu


def layout_model(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    """numpy model of the packed layout: tiles of 16 rows x 128 k, lane
    l = 16g + r holds bytes (2b, 2b+1) = canonical row 16t+r bytes
    64c + 8b + 2g + {0,1}; scale tile byte 8r + b = scale[16t+r][8c+b]."""
    NT, KT = -(-N // 16), -(-K // 128)
    cpad = np.zeros((NT * 16, KT * 64), np.uint8)
    cpad[:N, :K // 2] = codes
    spad = np.zeros((NT * 16, KT * 8), np.uint8)
    spad[:N, :K // 16] = scales
    pc = cpad.reshape(NT, 16, KT, 8, 4, 2).transpose(0, 2, 4, 1, 3, 5)   # t c g r b p
    ps = spad.reshape(NT, 16, KT, 8).transpose(0, 2, 1, 3)              # t c r b
    return pc.reshape(-1), ps.reshape(-1)


SHAPES = [(1, 16), (16, 128), (17, 144), (33, 400), (64, 256), (512, 256), (200, 1040),
          (48, 2064), (1, 4096)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_layout_and_roundtrip(N, K):
    m = q4()
    rng = np.random.default_rng(N * 7919 + K)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    note(f"pack N={N} K={K}")
    pc, ps = m.pack_weight(to_dev_u8(codes).reshape(-1), to_dev_u8(scales).reshape(-1), N, K)
    torch.cuda.synchronize()
    want_c, want_s = layout_model(codes, scales, N, K)
    assert np.array_equal(pc.cpu().numpy(), want_c)
    assert np.array_equal(ps.cpu().numpy(), want_s)
    # unpack into poisoned buffers: every byte must be rewritten
    c2 = torch.full((N * (K // 2),), 0xA5, dtype=torch.uint8, device=DEV)
    s2 = torch.full((N * (K // 16),), 0x5A, dtype=torch.uint8, device=DEV)
    note(f"unpack N={N} K={K}")
    m.q4proj_unpack(pc, ps, N, K, c2, s2)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy().reshape(N, K // 2), codes)
    assert np.array_equal(s2.cpu().numpy().reshape(N, K // 16), scales)


def test_pack_overwrites_padding_and_is_deterministic():
    m = q4()
    N, K = 21, 272
    rng = np.random.default_rng(5)
    codes = to_dev_u8(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)).reshape(-1)
    scales = to_dev_u8(rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)).reshape(-1)
    outs = []
    for fill in (0x00, 0xFF):
        pc = torch.full((m.q4proj_packed_codes_bytes(N, K),), fill, dtype=torch.uint8, device=DEV)
        ps = torch.full((m.q4proj_packed_scales_bytes(N, K),), fill, dtype=torch.uint8, device=DEV)
        note(f"pack fill={fill}")
        m.q4proj_pack(codes, scales, N, K, pc, ps)
        torch.cuda.synchronize()
        outs.append((pc.cpu().numpy(), ps.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408), (248320, 5120), (9216, 2560),
                                 (2560, 9216)])
def test_pack_roundtrip_full_size(N, K):
    """Every workload weight shape: device-side random bytes survive pack->unpack."""
    m = q4()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(N + K)
    codes = torch.randint(0, 256, (N * (K // 2),), dtype=torch.uint8, device=DEV, generator=gen)
    scales = torch.randint(0, 256, (N * (K // 16),), dtype=torch.uint8, device=DEV, generator=gen)
    note(f"pack full N={N} K={K}")
    pc, ps = m.pack_weight(codes, scales, N, K)
    c2 = torch.empty_like(codes)
    s2 = torch.empty_like(scales)
    m.q4proj_unpack(pc, ps, N, K, c2, s2)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scales)
    # a packed buffer holds exactly the input bytes plus zero padding
    assert int(pc.sum(dtype=torch.int64)) == int(codes.sum(dtype=torch.int64))
    assert int(ps.sum(dtype=torch.int64)) == int(scales.sum(dtype=torch.int64))
