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
    from ternary_weight_linear_act_amd import binding
    for want in ("bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_forward",
                 "bitlinear_packed_size", "bitlinear_last_error", "bitlinear_last_dispatch",
                 "bitlinear_forward_fused", "bitlinear_quant_act_ex", "bitlinear_forward_fused_ex",
                 "bitlinear_quant_act_h4", "bitlinear_forward_workspace_size", "bitlinear_forward_noalloc",
                 "bitlinear_forward_grouped", "bitlinear_quant_act_a48", "bitlinear_combine_a48",
                 "bitlinear_pack_weights_masked"):
        assert want in names
    # the binding's list is the header's
    assert sorted(binding.EXPORTED) == names


def test_exports_every_declared_symbol(lib):
    from ternary_weight_linear_act_amd import binding
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_allocates_no_device_memory():
    # the caller owns every buffer: the library imports no HIP allocator
    from ternary_weight_linear_act_amd import binding
    out = subprocess.run(["nm", "-D", "--undefined-only", binding.library_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = set(re.findall(r"\bU\s+(\S+)", out))
    for name in ("hipMalloc", "hipFree", "hipMallocAsync", "hipExtMallocWithFlags", "hipMallocManaged",
                 "hipHostMalloc", "hipMallocPitch"):
        assert not any(i.split("@")[0] == name for i in imported), name


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
                 a["acc"], a.get("work"), a.get("work_bytes", 0), None)

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
    assert call(work=P(8), work_bytes=1 << 20) == -1     # misaligned workspace


def work_size(lib, M, N, K, nm):
    from ternary_weight_linear_act_amd.binding import NM
    wb = ctypes.c_size_t(12345)
    st = lib.bitlinear_forward_workspace_size(M, N, K, NM(*nm), ctypes.byref(wb))
    return st, wb.value


def test_forward_workspace_size(lib):
    # no scratch: one token, the skinny kernels, the prefill tiles, the 2:4
    # sparse MFMA
    for (M, N, K, nm) in [(1, 6912, 2560, (0, 0)), (1, 2560, 6912, (6, 8)), (8, 2048, 11008, (0, 0)),
                          (64, 2048, 2048, (2, 4)), (2048, 6912, 2560, (0, 0)), (2048, 6912, 2560, (2, 4)),
                          (0, 6912, 2560, (6, 8))]:
        assert work_size(lib, M, N, K, nm) == (0, 0), (M, N, K, nm)
    # N:M rows expanded to dense codes at 65+ tokens off the sparse MFMA:
    # N * K / 4 bytes rounded up to 256 (plus the partial tiles when the
    # dense GEMM on them splits K)
    assert work_size(lib, 512, 8960, 1536, (6, 8)) == (0, 8960 * 1536 // 4)
    assert work_size(lib, 100, 4100, 192, (2, 4)) == (0, -(-4100 * 192 // 4 // 256) * 256)
    rows = -(-512 * 6912 // 4 // 256) * 256
    assert work_size(lib, 600, 512, 6912, (6, 8)) == (0, rows + 13 * 20 * 128 * 128 * 4)   # 13 splits of 20 tiles
    # past 64 tokens with fewer than 128 tiles of 128 x 128: K split
    assert work_size(lib, 512, 2560, 6912, (0, 0)) == (0, 4 * 80 * 128 * 128 * 4)
    # a few-token GEMM splitting K: 64 x 64 tiles (K > 4096, N < 8192), 64
    # tiles, 4 splits of 64 * 64 * 64 int32 partials
    assert work_size(lib, 40, 4096, 8192, (0, 0)) == (0, 4 * 64 * 64 * 64 * 4)
    # split partials stay within 32 MiB
    for M in (17, 33, 64):
        for N in (8192, 30000):
            st, wb = work_size(lib, M, N, 2048, (0, 0))
            assert st == 0 and wb <= 32 << 20
    assert work_size(lib, 4, 64, 100, (0, 0))[0] == -1        # K % 64
    assert work_size(lib, 4, 64, 128, (3, 4))[0] == -2
    from ternary_weight_linear_act_amd.binding import NM
    assert lib.bitlinear_forward_workspace_size(4, 64, 128, NM(0, 0), None) == -1


def test_forward_short_workspace_is_rejected_on_the_host(lib):
    # ESIZE before anything is launched: fake device addresses are never
    # touched
    from ternary_weight_linear_act_amd.binding import NM
    f = lib.bitlinear_forward
    need = work_size(lib, 512, 8960, 1536, (6, 8))[1]
    assert f(P(), P(), P(), P(), P(), NM(6, 8), 512, 8960, 1536, P(), None, P(), need - 1, None) == -3
    assert b"needed" in lib.bitlinear_last_error()
    assert f(P(), P(), P(), P(), P(), NM(6, 8), 512, 8960, 1536, P(), None, None, 0, None) == -3
    need = work_size(lib, 40, 4096, 8192, (0, 0))[1]
    assert f(P(), P(), P(), P(), P(), NM(0, 0), 40, 4096, 8192, P(), None, P(), need - 16, None) == -3


def test_noalloc_validation(lib):
    # host-side checks of the no-allocation forward: nothing reaches the GPU
    from ternary_weight_linear_act_amd.binding import NM
    f = lib.bitlinear_forward_noalloc
    assert f(None, P(), P(), P(), P(), NM(0, 0), 4, 8, 64, P(), None, None) == -1
    assert f(P(), P(), P(), P(), P(), NM(0, 0), 4, 8, 100, P(), None, None) == -1
    assert f(P(), P(), P(), P(), P(), NM(2, 8), 4, 8, 64, P(), None, None) == -2
    assert f(None, None, None, P(), P(), NM(0, 0), 0, 8, 64, None, None, None) == 0
    # more scratch than the fixed array holds (6:8 rows expanded: 64 MiB)
    assert f(P(), P(), P(), P(), P(), NM(6, 8), 100, 16384, 16384, P(), None, None) == -3
    assert b"32" in lib.bitlinear_last_error() or b"33554432" in lib.bitlinear_last_error()


def test_grouped_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM, Proj
    f = lib.bitlinear_forward_grouped
    arr = (Proj * 9)(*[Proj(A, A, 64, A, None) for _ in range(9)])
    assert f(P(), P(), P(), 4, 128, NM(0, 0), None, 1, None) == -1           # projs NULL
    assert f(P(), P(), P(), 4, 128, NM(0, 0), arr, 0, None) == -1            # nproj 0
    assert f(P(), P(), P(), 4, 128, NM(0, 0), arr, 9, None) == -2            # too many projections
    assert f(P(), P(), None, 4, 128, NM(0, 0), arr, 1, None) == -1           # row sums required
    assert f(P(8), P(), P(), 4, 128, NM(0, 0), arr, 1, None) == -1           # misaligned Xq
    assert f(P(), P(), P(), 4, 100, NM(0, 0), arr, 1, None) == -1            # K % 64
    assert f(P(), P(), P(), 65, 128, NM(0, 0), arr, 1, None) == -2           # M > 64
    big = (Proj * 2)(Proj(A, A, 11008, A, None), Proj(A, A, 11008, A, None))
    # past the skinny tiles' workgroups, the token-tile kernel's K (48 chunks)
    # and what the grouped GEMM takes: one projection, an N:M pattern, or
    # K > 4096 with fewer than 8192 rows
    assert f(P(), P(), P(), 64, 4096, NM(0, 0), big, 1, None) == -2
    assert f(P(), P(), P(), 64, 2048, NM(2, 4), big, 2, None) == -2
    deep = (Proj * 2)(Proj(A, A, 4096, A, None), Proj(A, A, 4096, A, None))
    assert f(P(), P(), P(), 64, 8192, NM(0, 0), deep, 2, None) == -2
    assert f(None, None, None, 0, 128, NM(0, 0), arr, 1, None) == 0          # M = 0: no-op


def test_a48_validation(lib):
    q = lib.bitlinear_quant_act_a48
    assert q(P(), 2, 256, -1, P(), P(), P(), None) == -1         # negative outlier count
    assert q(P(), 2, 256, 257, P(), P(), P(), None) == -1        # more outliers than inputs
    assert q(P(), 2, 16448, 10, P(), P(), P(), None) == -2       # K > 16384
    assert q(P(4), 2, 256, 3, P(), P(), P(), None) == -1         # misaligned X
    assert q(P(), 2, 100, 3, P(), P(), P(), None) == -1          # K % 64
    assert q(None, 0, 256, 3, None, None, None, None) == 0       # M = 0
    c = lib.bitlinear_combine_a48
    assert c(None, 2, 8, P(), None) == -1
    assert c(P(), 2, 0, P(), None) == -1
    assert c(None, 0, 8, None, None) == 0


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


def test_pack_masked_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM
    p = lib.bitlinear_pack_weights_masked
    assert p(P(), 8, 64, NM(0, 0), P(), 8 * 16, P(), P(), 256, None) == -1      # needs an N:M pattern
    assert p(P(), 8, 64, NM(3, 6), P(), 8 * 16, P(), P(), 256, None) == -2      # M not 4, 8 or 16
    assert p(P(), 8, 64, NM(9, 8), P(), 8 * 16, P(), P(), 256, None) == -2      # N > M
    assert p(P(), 8, 64, NM(0, 8), P(), 8 * 16, P(), P(), 256, None) == -2      # N = 0
    assert p(P(), 8, 64, NM(6, 8), P(), 8 * 16 - 1, P(), P(), 256, None) == -3  # dense layout: N*K/4 bytes
    assert p(P(), 8, 64, NM(6, 8), P(), 8 * 16, P(), P(), 8, None) == -3        # workspace
    assert p(P(4), 8, 64, NM(2, 4), P(), 8 * 16, P(), P(), 256, None) == -1     # misaligned W


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
    assert f(P(), 17, 128, NM(0, 0), arr, 1, None, None) == -2           # M > 16: use the two-call path
    assert f(P(), 2, 16384 + 64, NM(0, 0), arr, 1, None, None) == -2     # shared row too large
    assert f(P(), 9, 16384 + 64, NM(0, 0), arr, 1, None, None) == -2
    assert f(P(4), 1, 128, NM(0, 0), arr, 1, None, None) == -1           # misaligned X
    assert f(P(), 1, 128, NM(3, 4), arr, 1, None, None) == -2
    bad = (Proj * 1)(Proj(A + 4, A, 64, A, None))
    assert f(P(), 1, 128, NM(0, 0), bad, 1, None, None) == -1            # misaligned packed
    assert f(None, 0, 128, NM(0, 0), arr, 1, None, None) == 0            # M = 0: no-op


def test_fused_multi_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM, Proj, InputGroup
    f = lib.bitlinear_forward_fused_multi
    arr = (Proj * 9)(*[Proj(A, A, 64, A, None) for _ in range(9)])

    def groups(*gs):
        return (InputGroup * max(len(gs), 1))(*[InputGroup(x, k, a, n, xs) for (x, k, a, n, xs) in gs])
    ok = (P(), 128, arr, 1, None)
    assert f(None, 1, NM(0, 0), None) == -1                                   # groups NULL
    assert f(groups(ok), 0, NM(0, 0), None) == -1                             # ngroups 0
    assert f(groups(*[ok] * 5), 5, NM(0, 0), None) == -2                      # more than 4 groups
    assert f(groups(ok), 1, NM(3, 4), None) == -2                             # unsupported N:M
    assert f(groups(ok, (P(4), 128, arr, 1, None)), 2, NM(0, 0), None) == -1  # misaligned X
    assert f(groups(ok, (P(), 100, arr, 1, None)), 2, NM(0, 0), None) == -1   # K not a multiple of 64
    assert f(groups(ok, (P(), 65344 + 64, arr, 1, None)), 2, NM(0, 0), None) == -2   # K past one token's range
    assert f(groups(ok, (P(), 128, None, 1, None)), 2, NM(0, 0), None) == -1  # projs NULL
    assert f(groups(ok, (P(), 128, arr, 0, None)), 2, NM(0, 0), None) == -1   # nproj 0
    assert f(groups(ok, (P(), 128, arr, 9, None)), 2, NM(0, 0), None) == -2   # too many projections
    assert f(groups(ok, (P(), 128, arr, 1, P(2))), 2, NM(0, 0), None) == -1   # misaligned x_scale
    bad = (Proj * 1)(Proj(A, A, 64, None, None))
    assert f(groups(ok, (P(), 128, bad, 1, None)), 2, NM(0, 0), None) == -1   # Y NULL


def test_quant_multi_validation(lib):
    from ternary_weight_linear_act_amd.binding import QuantGroup
    f = lib.bitlinear_quant_act_multi

    def groups(*gs):
        return (QuantGroup * max(len(gs), 1))(*[QuantGroup(*g) for g in gs])
    ok = (P(), 2, 128, P(), P(), P())
    assert f(None, 1, None) == -1                                             # groups NULL
    assert f(groups(ok), 0, None) == -1                                       # ngroups 0
    assert f(groups(*[ok] * 9), 9, None) == -2                                # more than 8 groups
    assert f(groups(ok, (P(4), 2, 128, P(), P(), P())), 2, None) == -1        # misaligned X
    assert f(groups(ok, (P(), 2, 100, P(), P(), P())), 2, None) == -1         # K not a multiple of 64
    assert f(groups(ok, (P(), -1, 128, P(), P(), P())), 2, None) == -1        # negative M
    assert f(groups(ok, (P(), 2, 128, None, P(), P())), 2, None) == -1        # Xq NULL
    assert f(groups(ok, (P(), 2, 128, P(), P(2), P())), 2, None) == -1        # misaligned x_scale
    assert f(groups(ok, (P(), 2, 128, P(), P(), P(2))), 2, None) == -1        # misaligned x_rowsum


def test_grouped_multi_validation(lib):
    from ternary_weight_linear_act_amd.binding import NM, Proj, ActGroup
    f = lib.bitlinear_forward_grouped_multi
    arr = (Proj * 9)(*[Proj(A, A, 64, A, None) for _ in range(9)])

    def groups(*gs):
        return (ActGroup * max(len(gs), 1))(*[ActGroup(*g) for g in gs])
    ok = (P(), P(), P(), 2048, arr, 1)
    assert f(None, 1, 8, NM(0, 0), None) == -1                                     # groups NULL
    assert f(groups(ok), 0, 8, NM(0, 0), None) == -1                               # ngroups 0
    assert f(groups(*[ok] * 5), 5, 8, NM(0, 0), None) == -2                        # more than 4 groups
    assert f(groups(ok), 1, 8, NM(3, 4), None) == -2                               # unsupported N:M
    assert f(groups(ok), 1, 8, NM(2, 4), None) == -2                               # N:M weights
    assert f(groups(ok), 1, 4, NM(0, 0), None) == -2                               # M below 5
    assert f(groups(ok), 1, 9, NM(0, 0), None) == -2                               # M above 8
    assert f(groups(ok), 1, -1, NM(0, 0), None) == -1                              # negative M
    assert f(groups(ok, (P(4), P(), P(), 2048, arr, 1)), 2, 8, NM(0, 0), None) == -1   # misaligned Xq
    assert f(groups(ok, (P(), P(), P(), 100, arr, 1)), 2, 8, NM(0, 0), None) == -1     # K not a multiple of 64
    assert f(groups(ok, (P(), P(), P(), 12352, arr, 1)), 2, 8, NM(0, 0), None) == -2   # K past 12288
    assert f(groups(ok, (P(), P(), P(), 2048, arr, 9)), 2, 8, NM(0, 0), None) == -2    # too many projections
    assert f(groups(ok, (P(), P(), None, 2048, arr, 1)), 2, 8, NM(0, 0), None) == -1   # x_rowsum NULL
    assert f(groups(ok), 1, 0, NM(0, 0), None) == 0                                # M = 0: no-op


def test_trit24_sizes_and_validation(lib):
    # the trit-packed 2:4 layout: 12 bytes per 64 weights, as the oracle's
    # layout arithmetic counts them
    import oracle
    pb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    for (N, K) in [(8960, 1536), (1, 64), (3, 192), (2560, 6912)]:
        assert lib.bitlinear_packed_size_trit24(N, K, ctypes.byref(pb), ctypes.byref(wb)) == 0
        assert pb.value == oracle.packed_bytes_trit24(N, K) == 3 * N * K // 16
        assert wb.value == -(-8 * N // 256) * 256
    assert lib.bitlinear_packed_size_trit24(8, 96, None, None) == -1          # K % 64
    assert lib.bitlinear_packed_size_trit24(0, 64, None, None) == -1          # N < 1
    p = lib.bitlinear_pack_weights_trit24
    assert p(P(), 8, 64, P(), 8 * 12 - 1, P(), P(), 256, None) == -3          # packed one byte short
    assert p(P(), 8, 64, P(), 8 * 12, P(), P(), 8, None) == -3                # workspace short
    assert p(P(), 8, 64, P(), 8 * 12, P(), None, 256, None) == -1             # workspace missing
    assert p(P(4), 8, 64, P(), 8 * 12, P(), P(), 256, None) == -1             # misaligned W
    assert p(P(), 8, 100, P(), 8 * 12, P(), P(), 256, None) == -1             # K % 64


def test_trit24_forward_workspace_and_validation(lib):
    ws = ctypes.c_size_t(0)

    def need(M, N, K):
        st = lib.bitlinear_forward_trit24_workspace_size(M, N, K, ctypes.byref(ws))
        return st, ws.value
    # one token on the table-lookup kernel: no scratch up to K = 16384
    assert need(1, 8960, 1536) == (0, 0)
    assert need(1, 100, 16384) == (0, 0)
    assert need(0, 100, 1536) == (0, 0)
    # otherwise the rows expanded to dense codes (N * K / 4 rounded up to
    # 256) plus what the dense forward needs for the shape
    rows = -(-8960 * 1536 // 4 // 256) * 256
    assert need(512, 8960, 1536) == (0, rows + work_size(lib, 512, 8960, 1536, (0, 0))[1])
    assert need(5, 8960, 1536) == (0, rows + work_size(lib, 5, 8960, 1536, (0, 0))[1])
    rows = -(-40 * 16448 // 4 // 256) * 256
    assert need(1, 40, 16448) == (0, rows + work_size(lib, 1, 40, 16448, (0, 0))[1])
    rows = -(-2560 * 6912 // 4 // 256) * 256
    assert need(512, 2560, 6912) == (0, rows + 4 * 80 * 128 * 128 * 4)     # the dense GEMM splits K
    assert need(4, 64, 100)[0] == -1
    assert lib.bitlinear_forward_trit24_workspace_size(4, 64, 128, None) == -1
    f = lib.bitlinear_forward_trit24
    # a short workspace is ESIZE before anything is launched
    n = need(512, 8960, 1536)[1]
    assert f(P(), P(), P(), P(), P(), 512, 8960, 1536, P(), None, P(), n - 1, None) == -3
    assert b"needed" in lib.bitlinear_last_error()
    assert f(P(), P(), P(), P(), P(), 512, 8960, 1536, P(), None, None, 0, None) == -3
    # M == 0 is a no-op with NULL token buffers
    assert f(None, None, None, P(), P(), 0, 8960, 1536, None, None, None, 0, None) == 0
    assert lib.bitlinear_last_dispatch() == b"none"
    assert f(P(), P(), None, P(), P(), 1, 64, 64, P(), None, None, 0, None) == -1     # x_rowsum required
    assert f(P(), P(), P(), P(4), P(), 1, 64, 64, P(), None, None, 0, None) == -1     # misaligned packed
    assert f(P(), P(), P(), P(), P(), 1, 64, 64, P(), P(4), None, 0, None) == -1      # misaligned acc
    assert f(P(), P(), P(), P(), P(), 1, 0, 64, P(), None, None, 0, None) == -1       # N < 1
