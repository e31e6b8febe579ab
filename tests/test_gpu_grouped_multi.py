"""GPU parity of the grouped forward over several quantised inputs in one
launch (bitlinear_forward_grouped_multi, 5-8 tokens): every projection's acc
bit-exact against the CPU oracle and bit-identical to its own forward, Y
within the tolerance; the unsupported shapes raise."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_forward, hip_pack, to_dev

pytestmark = pytest.mark.gpu


def run(groups):
    """groups: list of (Ws, X) with X of M x K; one quant_act_multi, then
    one forward_grouped_multi."""
    import torch
    import ternary_weight_linear_act_amd as bl
    qcall, call, outs = [], [], []
    for Ws, X in groups:
        M, K = X.shape
        packs = [hip_pack(W, (0, 0)) for W in Ws]
        Xd = to_dev(X)
        Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        rs = torch.empty(M, dtype=torch.int32, device="cuda")
        Ys = [torch.full((M, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda") for W in Ws]
        accs = [torch.full((M, W.shape[0]), -7, dtype=torch.int32, device="cuda") for W in Ws]
        qcall.append((Xd, Xq, xs, rs))
        call.append((Xq, xs, rs, [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], Ys, accs))
        outs.append((packs, Xq, xs, rs, Ys, accs))
    bl.quant_act_multi(qcall)
    bl.forward_grouped_multi(call)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    return outs, call, name


def check(groups, outs):
    import torch
    import oracle
    for (Ws, X), (packs, Xq, xs, rs, Ys, accs) in zip(groups, outs):
        q, xs_o, _ = oracle.quant_act(X)
        assert np.array_equal(Xq.cpu().numpy(), q)
        for W, (pk, ws), Y, acc in zip(Ws, packs, Ys, accs):
            beta, w_eff, _ = oracle.quantize_weights(W)
            acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
            assert np.array_equal(acc.cpu().numpy(), acc_o)
            check_y(Y.cpu().numpy(), Y_o, acc_o)
            Y1, acc1 = hip_forward(Xq, xs, rs, pk, ws, W.shape[0], (0, 0))
            torch.cuda.synchronize()
            assert torch.equal(acc1, acc) and torch.equal(Y1.view(torch.int32), Y.view(torch.int32))


def test_block_3b_at_8_tokens_in_two_launches():
    d = workloads.draw("block_3b", Ms=(8,))
    gs = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    groups = [([d.W[n] for n in g], d.X[(g[0], 8)]) for g in gs]
    print("case grouped multi block_3b M=8", flush=True)
    outs, call, name = run(groups)
    assert name.startswith("skinny_direct_multi_dense") and name.count("+") == 3, name
    check(groups, outs)


# every configuration of the menu: K of 4-32 chunks (256, 2048; from 8192 rows
# two row blocks per wave), 33-40 (2304, 2560), 41-192 (2624, 6912, 12288);
# ragged weight rows
MULTI_CASES = [
    (5, [(256, (37,)), (2048, (300, 17)), (2304, (129,))]),
    (6, [(2048, (8200,)), (2560, (64, 65)), (2624, (33,))]),
    (7, [(6912, (100,)), (12288, (48,)), (1024, (1, 2, 3))]),
    (8, [(12288, (16,)), (256, (8192,))]),
]


@pytest.mark.parametrize("case", range(len(MULTI_CASES)))
def test_grouped_multi_shapes(case):
    M, spec = MULTI_CASES[case]
    groups = []
    for gi, (K, Ns) in enumerate(spec):
        seed = 4000 + 31 * case + 7 * gi + K
        Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
        _, X = workloads.small_case(seed + 99, M, 8, K, outlier_frac=0.01)
        groups.append((Ws, X))
    print("case grouped multi M=%d %s" % (M, spec), flush=True)
    outs, call, name = run(groups)
    assert name.startswith("skinny_direct_multi_dense"), name
    check(groups, outs)


# 9-64 tokens, the token-tile kernel's configurations <TT, RG, S>: <1,2,2>
# and <1,2,3> (K up to 32 chunks, then to 48), <1,4,2> and <1,4,3> (from
# 13824 rows at 17-32 tokens, 6912-13823 rows at 33-64), <2,6,2> (from 16384
# rows at 33-64 tokens, K <= 2048); ragged rows and token counts
TILES_CASES = [
    (9, [(2048, (7000,)), (2560, (6912,))]),
    (24, [(2048, (14000,)), (3072, (3000,)), (1024, (2600,))]),
    (40, [(2560, (7000,)), (1024, (16400,))]),
    (17, [(2048, (3000, 100)), (3072, (6912, 7000))]),
]


@pytest.mark.parametrize("case", range(len(TILES_CASES)))
def test_grouped_multi_token_tiles(case):
    M, spec = TILES_CASES[case]
    groups = []
    for gi, (K, Ns) in enumerate(spec):
        seed = 4500 + 31 * case + 7 * gi + K
        Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
        _, X = workloads.small_case(seed + 99, M, 8, K, outlier_frac=0.01)
        groups.append((Ws, X))
    print("case grouped multi tiles M=%d %s" % (M, spec), flush=True)
    outs, call, name = run(groups)
    assert name.startswith("skinny_direct_tiles_multi_dense"), name
    check(groups, outs)


def test_block_3b_at_64_tokens_shallow_groups():
    # q k v, o and gate up of the 3B block at 64 tokens in one launch (down,
    # K = 11008, is past the token-tile kernel's K)
    d = workloads.draw("block_3b", projs=["q", "k", "v", "o", "gate", "up"], Ms=(64,))
    gs = [("q", "k", "v"), ("o",), ("gate", "up")]
    groups = [([d.W[n] for n in g], d.X[(g[0], 64)]) for g in gs]
    print("case grouped multi block_3b M=64", flush=True)
    outs, call, name = run(groups)
    assert name.startswith("skinny_direct_tiles_multi_dense") and name.count("+") == 2, name
    check(groups, outs)


@pytest.mark.parametrize("M,K,nm", [(4, 2048, (0, 0)), (8, 192, (0, 0)), (8, 12352, (0, 0)), (8, 2048, (2, 4)),
                                    (9, 2048, (0, 0)), (64, 11008, (0, 0)), (65, 2048, (0, 0))])
def test_grouped_multi_unsupported(M, K, nm):
    import torch
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(4100 + M + K, M, 64, K)
    pk, ws = hip_pack(W, nm)
    Xq, xs, rs = bl.quant_act(to_dev(X))
    Y = torch.empty((M, 64), dtype=torch.float32, device="cuda")
    print("case grouped multi unsupported M=%d K=%d nm=%s" % (M, K, nm), flush=True)
    with pytest.raises(bl.BitLinearError) as e:
        bl.forward_grouped_multi([(Xq, xs, rs, [(pk, ws, 64)], [Y], None)], nm=nm)
    assert e.value.status == bl.binding.EUNSUPPORTED


def test_grouped_multi_graph_replay():
    import torch
    import ternary_weight_linear_act_amd as bl
    M = 8
    groups = [([workloads.small_case(4200, 1, 700, 2048)[0]], workloads.small_case(4201, M, 8, 2048)[1]),
              ([workloads.small_case(4202, 1, 300, 11008)[0]], workloads.small_case(4203, M, 8, 11008)[1])]
    print("case grouped multi graph", flush=True)
    outs, call, name = run(groups)
    check(groups, outs)
    ref = [[y.clone() for y in o[4]] for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            bl.forward_grouped_multi(call)
    torch.cuda.synchronize()
    for _ in range(3):
        for o in outs:
            for y in o[4]:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, o in zip(ref, outs):
            for a, b in zip(r, o[4]):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_grouped_multi_eight_projections_without_accumulators():
    import torch
    import oracle
    import ternary_weight_linear_act_amd as bl
    M, K = 6, 2048
    Ns = (16, 17, 100, 255, 256, 257, 31, 64)
    Ws = [workloads.small_case(4300 + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(4330, M, 8, K, outlier_frac=0.01)
    packs = [hip_pack(W, (0, 0)) for W in Ws]
    Xq, xs, rs = bl.quant_act(to_dev(X))
    Ys = [torch.full((M, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda") for W in Ws]
    print("case grouped multi 8 projections", flush=True)
    bl.forward_grouped_multi([(Xq, xs, rs, [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], Ys, None)])
    torch.cuda.synchronize()
    q, xs_o, _ = oracle.quant_act(X)
    for W, Y in zip(Ws, Ys):
        beta, w_eff, _ = oracle.quantize_weights(W)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        check_y(Y.cpu().numpy(), Y_o, acc_o)
