"""The C-ABI library on the CPU: it loads, exports every declared symbol, sizes
the packed layout, and rejects bad arguments on the host before touching a
device.  No projection is computed here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4proj.h")


@pytest.fixture(scope="module")
def q4():
    import nvfp4_weight_only_q4proj_amd as q4
    return q4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4proj_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(q4):
    names = declared_functions()
    assert len(names) == 19, names
    lib = q4.library()
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(q4.SYMBOLS) == names


def test_library_is_gfx950_only():
    # the shared object carries a gfx950 code object and no other GPU target
    data = open(os.path.join(ROOT, "nvfp4_weight_only_q4proj_amd", "libq4proj.so"), "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_"):
        assert b"amdgcn-amd-amdhsa--" + other not in data


@pytest.mark.parametrize("N,K", [(1, 16), (16, 128), (17, 144), (512, 256), (17408, 5120),
                                 (5120, 17408), (248320, 5120), (2560, 9216)])
def test_packed_sizes(q4, N, K):
    nt, kt = -(-N // 16), -(-K // 128)
    assert q4.q4proj_packed_codes_bytes(N, K) == nt * kt * 1024 >= N * K // 2
    assert q4.q4proj_packed_scales_bytes(N, K) == nt * kt * 128 >= N * K // 16
    # gemv's exchange words: one 64-bit word x 4 rows x 64 lanes per workgroup
    # boundary (256 at most), plus one word per output for each of the KS - 1
    # joins when K is cut into KS ranges; a range's activations (M x k-tiles
    # x 256 B / KS) must fit in the 147,392 staging bytes, and which of the
    # counts that fit is taken is the library's estimate (M = 1 takes one
    # range up to K = 65536; the verify shape M = 7, K = 17408 four)
    for M in (1, 7, 16):
        got = q4.q4proj_workspace_bytes(M, N, K)
        extra = got - 512 * 1024
        assert extra >= 0 and extra % (8 * M * N) == 0, (M, got)
        ks = extra // (8 * M * N) + 1
        assert ks in (1, 2, 4, 8) and M * -(-kt // ks) * 256 <= 147392, (M, ks)
        if M == 1:
            assert ks == 1
        if (M, N, K) == (7, 5120, 17408):
            assert ks == 4
    assert q4.q4proj_workspace_bytes(17, N, K) == 0
    assert q4.q4proj_workspace_bytes(512, N, K) == 0
    # the GEMMs' optional staging workspace: 2MK and 4M bytes, each rounded
    # up to 256
    for M in (1, 7, 512, 513):
        r256 = lambda n: -(-n // 256) * 256
        assert q4.q4proj_gemm_workspace_bytes(M, N, K) == r256(2 * M * K) + r256(4 * M)


def test_workspace_of_the_verify_shape(q4):
    # M = 7 at K = 17408 (down, 244 KB of activations): four K ranges, three
    # joins; at K = 5120 (gate/up) one range
    assert q4.q4proj_workspace_bytes(7, 5120, 17408) == 512 * 1024 + 3 * 8 * 7 * 5120
    assert q4.q4proj_workspace_bytes(7, 17408, 5120) == 512 * 1024


def fitting_ranges(M, K):
    """K range counts (1, 2, 4, 8, none of them empty) whose activations,
    M x k-tiles-per-range x 256 B, fit in the 147,392 staging bytes."""
    kt = -(-K // 128)
    out = []
    for ks in (1, 2, 4, 8):
        ktr = -(-kt // ks)
        if kt - (ks - 1) * ktr < 1:
            break
        if M * ktr * 256 <= 147392:
            out.append(ks)
    return out


@pytest.mark.parametrize("M", [1, 2, 7, 12, 13, 16])
@pytest.mark.parametrize("F,K", [(16, 16), (17408, 5120), (8192, 8192), (4096, 17408),
                                 (64, 32768), (64, 65536), (64, 262144)])
def test_silu_mul_workspace(q4, M, F, K):
    # served exactly when some range count fits; the workspace then holds the
    # boundary words plus M x F words per join of the count taken
    fits = fitting_ranges(M, K)
    got = q4.q4proj_silu_mul_workspace_bytes(M, F, K)
    if not fits:
        assert got == 0
        return
    extra = got - 8 * 65536
    assert extra >= 0 and extra % (8 * M * F) == 0, got
    assert extra // (8 * M * F) + 1 in fits


def test_silu_mul_workspace_limits(q4):
    # M = 16 is served while 16 x ceil(k-tiles / 8) x 256 <= 147,392 B, i.e.
    # up to 280 k-tiles
    assert q4.q4proj_silu_mul_workspace_bytes(16, 64, 280 * 128) > 0
    assert q4.q4proj_silu_mul_workspace_bytes(16, 64, 281 * 128) == 0
    assert q4.q4proj_silu_mul_workspace_bytes(1, 8, 128) == 8 * 65536     # one k-tile: one range
    for M, F, K in [(0, 16, 128), (17, 16, 128), (1, 4, 128), (1, 12, 128), (1, 0, 128),
                    (1, 16, 120), (1, 16, 0)]:
        assert q4.q4proj_silu_mul_workspace_bytes(M, F, K) == 0, (M, F, K)


@pytest.mark.parametrize("N,K", [(0, 16), (16, 0), (16, 8), (16, 24), (-1, 16)])
def test_packed_sizes_invalid(q4, N, K):
    assert q4.q4proj_packed_codes_bytes(N, K) == 0
    assert q4.q4proj_packed_scales_bytes(N, K) == 0


# Fake, well-aligned, non-overlapping addresses: every call below must be
# rejected by the host-side checks before any HIP call is made.
A, B, X, Y, W = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
WSB = 512 * 1024


def proj(lib, fn, pc=A, ps=B, x=X, y=Y, M=1, N=64, K=256, ws=W, wsb=WSB):
    return getattr(lib, fn)(pc, ps, ctypes.c_float(1.0), x, y, M, N, K, ws, wsb, None)


@pytest.mark.parametrize("fn", ["q4proj_gemv", "q4proj_gemm"])
def test_projection_validation(q4, fn):
    lib = q4.library()
    assert proj(lib, fn, pc=None) == q4.EINVAL
    assert proj(lib, fn, ps=None) == q4.EINVAL
    assert proj(lib, fn, x=None) == q4.EINVAL
    assert proj(lib, fn, y=None) == q4.EINVAL
    assert proj(lib, fn, M=0) == q4.EINVAL
    assert proj(lib, fn, N=0) == q4.EINVAL
    assert proj(lib, fn, K=0) == q4.EINVAL
    assert proj(lib, fn, K=24) == q4.EINVAL          # K % 16 != 0
    assert proj(lib, fn, M=-3) == q4.EINVAL
    assert proj(lib, fn, x=X + 8) == q4.EINVAL       # x must be 16-byte aligned
    assert proj(lib, fn, pc=A + 4) == q4.EINVAL
    assert proj(lib, fn, y=Y + 2) == q4.EINVAL
    assert proj(lib, fn, y=X + 64) == q4.EINVAL      # y overlaps x
    assert proj(lib, fn, y=A) == q4.EINVAL           # y overlaps the packed codes


def test_gemv_workspace_validation(q4):
    lib = q4.library()
    assert proj(lib, "q4proj_gemv", wsb=WSB - 8) == q4.EWORKSPACE
    assert proj(lib, "q4proj_gemv", ws=None, wsb=0) == q4.EWORKSPACE
    assert proj(lib, "q4proj_gemv", ws=None) == q4.EINVAL        # size given, no buffer
    assert proj(lib, "q4proj_gemv", ws=W + 4) == q4.EINVAL       # 8-byte alignment
    assert proj(lib, "q4proj_gemv", ws=Y - 4096) == q4.EINVAL    # overlaps y
    assert proj(lib, "q4proj_gemv", ws=X) == q4.EINVAL           # overlaps x


def test_gemm_workspace_validation(q4):
    # the optional staging workspace of the GEMMs: big enough, 16-byte
    # aligned, apart from every other argument
    lib = q4.library()
    need = q4.q4proj_gemm_workspace_bytes(512, 64, 256)
    assert need == 2 * 512 * 256 + 2048
    assert proj(lib, "q4proj_gemm", M=512, wsb=need - 1) == q4.EWORKSPACE
    assert proj(lib, "q4proj_gemm", M=512, ws=W + 8, wsb=need) == q4.EINVAL
    assert proj(lib, "q4proj_gemm", M=512, ws=X + 4096, wsb=need) == q4.EINVAL   # overlaps x
    assert proj(lib, "q4proj_gemm", M=512, ws=Y - 4096, wsb=need) == q4.EINVAL   # overlaps y
    assert proj(lib, "q4proj_gemm", M=512, ws=A, wsb=need) == q4.EINVAL          # packed codes
    assert silu(lib, fn="q4proj_gemm_silu_mul", M=512, wsb=need - 1) == q4.EWORKSPACE
    assert silu(lib, fn="q4proj_gemm_silu_mul", M=512, ws=Y, wsb=need) == q4.EINVAL  # overlaps h
    assert q4.q4proj_gemm_workspace_bytes(0, 64, 256) == 0
    assert q4.q4proj_gemm_workspace_bytes(1, 64, 250) == 0


def test_binding_stages_gemm_activations_where_it_pays(q4):
    # the binding's default GEMM call stages fp16 operands only where its
    # estimate says the kernel time saved exceeds the staging: at M = 512,
    # K = 5120 not for the qkv width, for gate/up and the fused pair; not at
    # small M, nor for the 17408-wide rows of the down projection at M = 512
    assert not q4.gemm_staging_pays(512, 14336, 5120)
    assert q4.gemm_staging_pays(512, 17408, 5120)
    assert q4.gemm_staging_pays(512, 34816, 5120)
    assert not q4.gemm_staging_pays(64, 17408, 5120)
    assert not q4.gemm_staging_pays(512, 5120, 17408)
    assert q4.gemm_staging_pays(4096, 14336, 5120)


def test_gemv_m_range(q4):
    lib = q4.library()
    assert proj(lib, "q4proj_gemv", M=17) == q4.EUNSUPPORTED
    assert proj(lib, "q4proj_gemv", M=1000) == q4.EUNSUPPORTED


def silu(lib, pc=A, ps=B, x=X, h=Y, M=1, F=64, K=256, ws=W, wsb=WSB, fn="q4proj_gemv_silu_mul"):
    return getattr(lib, fn)(pc, ps, ctypes.c_float(1.0), x, h, M, F, K, ws, wsb, None)


SILU_BAD = [dict(pc=None), dict(ps=None), dict(x=None), dict(h=None), dict(M=0), dict(F=0),
            dict(F=12), dict(F=-16), dict(K=0), dict(K=24), dict(x=X + 8), dict(pc=A + 4),
            dict(ps=B + 4), dict(h=Y + 1), dict(h=X + 64), dict(h=A), dict(M=-1)]


def test_silu_mul_validation(q4):
    lib = q4.library()
    assert q4.q4proj_silu_mul_workspace_bytes(1, 64, 256) == WSB
    for kw in SILU_BAD + [dict(ws=None), dict(ws=W + 4), dict(ws=Y - 4096), dict(ws=X)]:
        assert silu(lib, **kw) == q4.EINVAL, kw
    assert silu(lib, M=17) == q4.EUNSUPPORTED
    assert silu(lib, M=16, K=281 * 128) == q4.EUNSUPPORTED
    assert silu(lib, wsb=WSB - 8) == q4.EWORKSPACE
    assert silu(lib, ws=None, wsb=0) == q4.EWORKSPACE
    for kw in SILU_BAD:
        assert silu(lib, **{"fn": "q4proj_gemm_silu_mul", "M": 512, **kw}) == q4.EINVAL, kw


def test_argmax_validation(q4):
    lib = q4.library()
    need = q4.q4proj_argmax_workspace_bytes(1, 64, 256)
    assert need == 512 * 1024 + 16
    assert q4.q4proj_argmax_workspace_bytes(17, 64, 256) == 0
    assert q4.q4proj_argmax_workspace_bytes(16, 64, 281 * 128) == 0
    # the gemv workspace of the shape (four K ranges here) plus 8 * (M + 1) bytes
    assert q4.q4proj_argmax_workspace_bytes(7, 5120, 17408) == 512 * 1024 + 3 * 8 * 7 * 5120 + 64
    V, I = W + (1 << 20), W + (1 << 20) + 4096

    def am(pc=A, ps=B, x=X, y=Y, val=V, idx=I, M=1, N=64, K=256, ws=W, wsb=need):
        return lib.q4proj_gemv_argmax(pc, ps, ctypes.c_float(1.0), x, y, val, idx, M, N, K, ws,
                                      wsb, None)

    for kw in [dict(pc=None), dict(ps=None), dict(x=None), dict(val=None), dict(idx=None),
               dict(M=0), dict(N=0), dict(K=24), dict(x=X + 8), dict(y=Y + 2), dict(val=V + 2),
               dict(idx=I + 4), dict(y=X + 64), dict(val=A), dict(idx=V), dict(val=Y + 64),
               dict(ws=None), dict(ws=W + 4), dict(ws=X), dict(ws=V - 64)]:
        assert am(**kw) == q4.EINVAL, kw
    assert am(M=17) == q4.EUNSUPPORTED
    assert am(M=16, K=281 * 128) == q4.EUNSUPPORTED
    assert am(wsb=need - 8) == q4.EWORKSPACE
    assert am(ws=None, wsb=0) == q4.EWORKSPACE


def test_quantize_validation(q4):
    lib = q4.library()
    assert q4.q4proj_quantize_workspace_bytes(16, 128) == 4096
    assert q4.q4proj_quantize_workspace_bytes(16, 120) == 0
    assert q4.q4proj_quantize_workspace_bytes(0, 128) == 0
    C, S, G = X, Y, W + 65536

    def quant(w=A, N=16, K=128, codes=C, scales=S, g=G, ws=W, wsb=4096):
        return lib.q4proj_quantize(w, N, K, codes, scales, g, ws, wsb, None)

    for kw in [dict(w=None), dict(codes=None), dict(scales=None), dict(g=None), dict(N=0),
               dict(K=0), dict(K=24), dict(N=-1), dict(w=A + 8), dict(codes=C + 4), dict(g=G + 2),
               dict(codes=A), dict(scales=A + 64), dict(scales=C + 16), dict(g=S), dict(ws=None),
               dict(ws=W + 2), dict(ws=G - 16)]:
        assert quant(**kw) == q4.EINVAL, kw
    assert quant(wsb=4095) == q4.EWORKSPACE
    assert quant(ws=None, wsb=0) == q4.EWORKSPACE


@pytest.mark.parametrize("fn", ["q4proj_pack", "q4proj_unpack"])
def test_pack_validation(q4, fn):
    lib = q4.library()
    f = getattr(lib, fn)
    assert f(None, B, 16, 128, X, Y, None) == q4.EINVAL
    assert f(A, None, 16, 128, X, Y, None) == q4.EINVAL
    assert f(A, B, 16, 120, X, Y, None) == q4.EINVAL
    assert f(A, B, 0, 128, X, Y, None) == q4.EINVAL
    assert f(A, B, 16, 128, A, Y, None) == q4.EINVAL   # in place
    assert f(A, B, 16, 128, X + 4, Y, None) == q4.EINVAL


def test_pack_gate_up_validation(q4):
    """Fused gate/up pack: F a positive multiple of 8, equal (non-NaN) global
    scales, aligned and non-overlapping buffers; host checks only."""
    lib = q4.library()
    one = ctypes.c_float(1.0)

    def f(gc=A, gs=B, uc=A + 65536, us=B + 65536, g1=one, g2=one, F=16, K=128, pc=X, ps=Y):
        return lib.q4proj_pack_gate_up(gc, gs, uc, us, g1, g2, F, K, pc, ps, None)

    for kw in [dict(gc=None), dict(us=None), dict(pc=None), dict(F=0), dict(F=12), dict(F=4),
               dict(K=120), dict(K=0), dict(g2=ctypes.c_float(2.0)),
               dict(g1=ctypes.c_float(float("nan")), g2=ctypes.c_float(float("nan"))),
               dict(g1=ctypes.c_float(0.0), g2=ctypes.c_float(-0.0)),
               dict(gc=A + 4), dict(pc=X + 8), dict(ps=Y + 4), dict(pc=A), dict(ps=B + 65536),
               dict(ps=X)]:
        assert f(**kw) == q4.EINVAL, kw


def test_gemv_noalloc_validation(q4):
    """The allocation-free GEMV checks its arguments as q4proj_gemv does and
    refuses shapes whose exchange words exceed its 8 MiB array."""
    lib = q4.library()
    f = lib.q4proj_gemv_noalloc
    one = ctypes.c_float(1.0)
    assert f(None, B, one, X, Y, 1, 64, 256, None) == q4.EINVAL
    assert f(A, B, one, X, None, 1, 64, 256, None) == q4.EINVAL
    assert f(A, B, one, X, Y, 1, 64, 250, None) == q4.EINVAL
    assert f(A, B, one, X + 8, Y, 1, 64, 256, None) == q4.EINVAL
    assert f(A, B, one, X, Y, 17, 64, 256, None) == q4.EUNSUPPORTED
    # 16 rows on the lm-head shape: 512 KiB + 8 * 16 * 248320 B of words
    assert q4.q4proj_workspace_bytes(16, 248320, 5120) > 8 << 20
    assert f(A, B, one, X, W, 16, 248320, 5120, None) == q4.EWORKSPACE


def test_status_strings(q4):
    lib = q4.library()
    for s in range(6):
        assert lib.q4proj_status_string(s).decode().startswith("Q4P_")
    assert b"unknown" in lib.q4proj_status_string(99)


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="needs a host without a GPU")
def test_no_device_no_fallback(q4):
    """With valid arguments and no gfx950 device the library refuses (EDEVICE)
    instead of computing anything elsewhere."""
    lib = q4.library()
    assert proj(lib, "q4proj_gemv") == q4.EDEVICE
    assert proj(lib, "q4proj_gemm", M=512) == q4.EDEVICE
    assert proj(lib, "q4proj_gemm", M=512, ws=None, wsb=0) == q4.EDEVICE   # workspace optional
    assert proj(lib, "q4proj_gemm", M=512, ws=None, wsb=123) == q4.EDEVICE
    assert lib.q4proj_pack(A, B, 16, 128, X, Y, None) == q4.EDEVICE
    assert lib.q4proj_gemv_noalloc(A, B, ctypes.c_float(1.0), X, Y, 1, 64, 256, None) == q4.EDEVICE
    assert lib.q4proj_pack_gate_up(A, B, A + 65536, B + 65536, ctypes.c_float(0.5),
                                   ctypes.c_float(0.5), 16, 128, X, Y, None) == q4.EDEVICE
    assert silu(lib) == q4.EDEVICE
    assert silu(lib, h=Y + 2) == q4.EDEVICE             # bf16 out needs 2-byte alignment only
    assert silu(lib, fn="q4proj_gemm_silu_mul", M=512, ws=None, wsb=0) == q4.EDEVICE
    assert lib.q4proj_quantize(A, 16, 128, X, Y, W + 65536, W, 4096, None) == q4.EDEVICE
    assert lib.q4proj_gemv_argmax(A, B, ctypes.c_float(1.0), X, None, W + (1 << 20),
                                  W + (1 << 20) + 4096, 1, 64, 256, W, 512 * 1024 + 16,
                                  None) == q4.EDEVICE


def test_plain_c_consumer_builds(tmp_path):
    """The plain C consumer of the ABI (run on the GPU by test_gpu_c_abi.py)
    compiles against include/q4proj.h and links the library."""
    import importlib.util
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(here, "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = mod.build(out=str(tmp_path / "libabi_consumer.so"))
    # not loaded here: its run paths are relative to tests/c_abi/
    assert b"abi_consumer_run" in open(out, "rb").read()
