"""CPU-side checks of the C ABI: the library loads without a GPU, exports every
symbol include/bitlinear.h declares, reports sizes, and rejects bad arguments
on the host before anything reaches the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="module")
def lib():
    from ternary_weight_linear_act_amd import binding
    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_forward",
                 "bitlinear_packed_size", "bitlinear_last_error", "bitlinear_last_dispatch",
                 "bitlinear_forward_fused", "bitlinear_quant_act_ex", "bitlinear_forward_fused_ex",
                 "bitlinear_quant_act_h4"):
        assert want in names


def test_exports_every_declared_symbol(lib):
    from ternary_weight_linear_act_amd import binding
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "bitlinear.h"\nint main(void){bitlinear_nm nm={2,4};'
                   'size_t p=0;return (int)bitlinear_packed_size(8,64,nm,&p,0);}\n')
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-c", "-I", os.path.join(ROOT, "include"),
                           str(src), "-o", str(tmp_path / "t.o")])


def sizes(lib, N, K, nm):
    from ternary_weight_linear_act_amd.binding import NM
    pb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.bitlinear_packed_size(N, K, NM(*nm), ctypes.byref(pb), ctypes.byref(wb))
    return st, pb.value, wb.value


def test_packed_sizes(lib):
    assert sizes(lib, 6912, 2560, (0, 0)) == (0, 4423680, 55296)
    assert sizes(lib, 8960, 1536, (2, 4))[:2] == (0, 3440640)
    assert sizes(lib, 8960, 1536, (6, 8))[:2] == (0, 4300800)
    assert sizes(lib, 1, 64, (0, 0)) == (0, 16, 256)
    # the byte counts agree with the oracle's own layout arithmetic
    import oracle
    for (N, K, nm) in [(6912, 2560, (0, 0)), (8960, 1536, (2, 4)), (8960, 1536, (6, 8)), (3, 192, (6, 8))]:
        assert sizes(lib, N, K, nm)[1] == oracle.packed_bytes(N, K, *nm)


@pytest.mark.parametrize("N,K,nm,status", [
    (8, 96, (0, 0), -1),          # K % 64
    (8, 0, (0, 0), -1),
    (0, 64, (0, 0), -1),          # N < 1
    (8, 64, (3, 4), -2),          # unsupported pattern
    (8, 64, (4, 4), -2),
    (8, 64, (1, 1), -2),
    (8, 2 * 1048576, (0, 0), -1),  # K too large
])
def test_size_query_rejects(lib, N, K, nm, status):
    assert sizes(lib, N, K, nm)[0] == status
    assert lib.bitlinear_last_error()


# Fake but aligned device-looking addresses: every call below must be rejected
# by host-side validation, so nothing is ever dereferenced or launched.
A = 0x10000


def P(off=0):
    return ctypes.c_void_p(A + off)


def test_forward_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM
    f = lib.bitlinear_forward
    ok = dict(Xq=P(), xs=P(), rs=P(), packed=P(), ws=P(), nm=NM(0, 0), M=4, N=8, K=64, Y=P(), acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["Xq"], a["xs"], a["rs"], a["packed"], a["ws"], a["nm"], a["M"], a["N"], a["K"], a["Y"],
                 a["acc"], None)

    assert call(Xq=None) == -1
    assert call(rs=None) == -1                # the row sums are required
    assert call(Y=P(4)) == -1                 # misaligned output
    assert call(Xq=P(8)) == -1
    assert call(acc=P(4)) == -1
    assert call(K=100) == -1
    assert call(N=0) == -1
    assert call(M=-1) == -1
    assert call(nm=NM(2, 8)) == -2
    assert b"2:8" in lib.bitlinear_last_error()
    # M == 0 is a successful no-op that launches nothing
    assert call(M=0) == 0
    assert lib.bitlinear_last_dispatch() == b"none"
    assert call(M=0, Xq=None, xs=None, rs=None, Y=None) == 0     # M-sized buffers may be NULL
    assert call(M=0, packed=None) == -1


def test_quant_validation(lib):
    q = lib.bitlinear_quant_act
    assert q(None, 4, 64, P(), P(), P(), None) == -1
    assert q(P(4), 4, 64, P(), P(), P(), None) == -1
    assert q(P(), 4, 64, P(), P(), P(2), None) == -1
    assert q(P(), 4, 65, P(), P(), P(), None) == -1
    assert q(P(), -1, 64, P(), P(), P(), None) == -1
    assert q(P(), 0, 64, P(), P(), None, None) == 0
    assert q(None, 0, 64, None, None, None, None) == 0


def test_transform_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM, ActTransform, Proj
    q = lib.bitlinear_quant_act_ex
    ok = ActTransform(A, A, 1e-5)
    assert q(P(), ctypes.byref(ActTransform(A + 4, None, 0.0)), 4, 64, P(), P(), P(), None) == -1   # up misaligned
    assert q(P(), ctypes.byref(ActTransform(None, A + 8, 0.0)), 4, 64, P(), P(), P(), None) == -1   # gamma misaligned
    assert q(P(), ctypes.byref(ActTransform(None, A, -1.0)), 4, 64, P(), P(), P(), None) == -1      # eps < 0
    assert q(P(), ctypes.byref(ActTransform(None, A, float("nan"))), 4, 64, P(), P(), P(), None) == -1
    assert q(P(), ctypes.byref(ActTransform(None, A, float("inf"))), 4, 64, P(), P(), P(), None) == -1
    assert q(P(), ctypes.byref(ok), 4, 65, P(), P(), P(), None) == -1                               # bad K
    assert q(None, ctypes.byref(ok), 0, 64, None, None, None, None) == 0                            # M = 0
    f = lib.bitlinear_forward_fused_ex
    arr = (Proj * 1)(Proj(A, A, 64, A, None))
    assert f(P(), ctypes.byref(ok), 2, 128, NM(0, 0), arr, 1, None, None) == -2          # transform: M == 1 only
    assert f(P(), ctypes.byref(ok), 1, 16448, NM(0, 0), arr, 1, None, None) == -2        # ... and K <= 16384
    assert f(P(), ctypes.byref(ActTransform(None, A, -2.0)), 1, 128, NM(0, 0), arr, 1, None, None) == -1
    assert f(None, ctypes.byref(ok), 0, 128, NM(0, 0), arr, 1, None, None) == 0


def test_h4_validation(lib):
    q = lib.bitlinear_quant_act_h4
    assert q(P(), 2, 256, 3, P(), P(), P(), None) == -1          # block not a power of two
    assert q(P(), 2, 256, 512, P(), P(), P(), None) == -1        # block does not divide K
    assert q(P(), 2, 16384, 16384, P(), P(), P(), None) == -1    # block > 8192
    assert q(P(), 2, 256, 0, P(), P(), P(), None) == -1
    assert q(P(4), 2, 256, 64, P(), P(), P(), None) == -1        # misaligned X
    assert q(None, 0, 256, 64, None, None, None, None) == 0      # M = 0


def test_pack_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM
    p = lib.bitlinear_pack_weights
    # packed buffer one byte short
    assert p(P(), 8, 64, NM(0, 0), P(), 8 * 16 - 1, P(), P(), 256, None) == -3
    # workspace too small
    assert p(P(), 8, 64, NM(0, 0), P(), 8 * 16, P(), P(), 8, None) == -3
    # workspace missing
    assert p(P(), 8, 64, NM(0, 0), P(), 8 * 16, P(), None, 256, None) == -1
    assert p(P(), 8, 64, NM(6, 8), P(), 8 * 16, P(), P(), 256, None) == -3   # 6:8 needs 5/16 bytes per weight
    assert p(P(), 8, 64, NM(7, 8), P(), 8 * 16, P(), P(), 256, None) == -2
    assert p(None, 8, 64, NM(0, 0), P(), 8 * 16, P(), P(), 256, None) == -1


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    from ternary_weight_linear_act_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library()


def test_fused_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM, Proj
    f = lib.bitlinear_forward_fused
    arr = (Proj * 9)(*[Proj(A, A, 64, A, None) for _ in range(9)])
    assert f(P(), 1, 128, NM(0, 0), None, 1, None, None) == -1           # projs NULL
    assert f(P(), 1, 128, NM(0, 0), arr, 0, None, None) == -1            # nproj 0
    assert f(P(), 1, 128, NM(0, 0), arr, 9, None, None) == -2            # too many projections
    assert f(P(), 5, 128, NM(0, 0), arr, 1, None, None) == -2            # M > 4: use the two-call path
    assert f(P(), 2, 16384 + 64, NM(0, 0), arr, 1, None, None) == -2     # shared row too large
    assert f(P(4), 1, 128, NM(0, 0), arr, 1, None, None) == -1           # misaligned X
    assert f(P(), 1, 128, NM(3, 4), arr, 1, None, None) == -2
    bad = (Proj * 1)(Proj(A + 4, A, 64, A, None))
    assert f(P(), 1, 128, NM(0, 0), bad, 1, None, None) == -1            # misaligned packed
    assert f(None, 0, 128, NM(0, 0), arr, 1, None, None) == 0            # M = 0: no-op
