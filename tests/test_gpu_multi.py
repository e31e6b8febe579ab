"""GPU parity of the one-token decode over several input groups in one launch
(bitlinear_forward_fused_multi): every group's codes, scale, accumulators and
outputs against the CPU oracle, and bit-identical to that group's own
forward_fused call."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_pack, to_dev

pytestmark = pytest.mark.gpu


def run_multi(groups, nm=(0, 0)):
    """groups: list of (Ws, X); returns per group (packs, Ys, accs, xs) and
    the dispatch name."""
    import torch
    import ternary_weight_linear_act_amd as bl
    out, call = [], []
    for Ws, X in groups:
        packs = [hip_pack(W, nm) for W in Ws]
        Xd = to_dev(X)
        Ys = [torch.full((1, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda") for W in Ws]
        accs = [torch.full((1, W.shape[0]), -7, dtype=torch.int32, device="cuda") for W in Ws]
        xs = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        out.append((packs, Ys, accs, xs))
        call.append((Xd, [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], Ys, accs, xs))
    bl.forward_fused_multi(call, nm=nm)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    return out, call, name


def check_group(Ws, X, nm, Ys, accs, xs):
    import oracle
    q, xs_o, _ = oracle.quant_act(X)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
    for W, Y, acc in zip(Ws, Ys, accs):
        beta, w_eff, _ = oracle.quantize_weights(W, *nm)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        check_y(Y.cpu().numpy(), Y_o, acc_o)


def check_same_as_single(call, out, nm):
    """Each group's results equal its own forward_fused call, bit for bit."""
    import torch
    import ternary_weight_linear_act_amd as bl
    for (Xd, projs, _, _, _), (_, Ys, accs, xs) in zip(call, out):
        xs1 = torch.empty(1, dtype=torch.float32, device="cuda")
        Ys1, accs1 = bl.forward_fused(Xd, projs, nm, want_acc=True, x_scale=xs1)
        torch.cuda.synchronize()
        assert torch.equal(xs1.view(torch.int32), xs.view(torch.int32))
        for a, b in zip(Ys1, Ys):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        for a, b in zip(accs1, accs):
            assert torch.equal(a, b)


def test_decode_ffn_2b_one_launch():
    # gate and up share one input, down has its own: the decode step's
    # three projections in one launch
    d = workloads.draw("decode_ffn_2b")
    groups = [([d.W["gate"], d.W["up"]], d.X[("gate", 1)]), ([d.W["down"]], d.X[("down", 1)])]
    print("case multi decode_ffn_2b", flush=True)
    out, call, name = run_multi(groups)
    assert name.startswith("fused_decode_multi_dense"), name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)
    check_same_as_single(call, out, (0, 0))


def test_decode_ffn_2b_down_first():
    d = workloads.draw("decode_ffn_2b")
    groups = [([d.W["down"]], d.X[("down", 1)]), ([d.W["gate"], d.W["up"]], d.X[("gate", 1)])]
    print("case multi decode_ffn_2b down first", flush=True)
    out, call, name = run_multi(groups)
    assert name.startswith("fused_decode_multi_dense"), name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)


def test_block_3b_m1_one_launch():
    # the block's four input groups: q k v, o, gate up, down (three
    # configurations of the kernel's menu in one grid)
    d = workloads.draw("block_3b", Ms=(1,))
    gs = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    groups = [([d.W[n] for n in g], d.X[(g[0], 1)]) for g in gs]
    print("case multi block_3b M=1", flush=True)
    out, call, name = run_multi(groups)
    assert name.startswith("fused_decode_multi_dense") and name.count("+") == 3, name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)
    check_same_as_single(call, out, (0, 0))


# K values that reach every class of the kernel's menu: 4 lanes per row for
# K <= 2048 (64, 256: 1 chunk per lane; 320: 2; 640: 3; 1024: 4; 1280: 5;
# 1536: 6; 1792: 7; 2048: 8 in the block above), with 6 waves for 13000 rows
# of 1024 and 8 for the 3B gate+up; past that the one-input rule: 8 lanes
# (2304, 2560: 5 chunks; 3072: 6; 3584: 7; 8 waves for 2 x 6912 and 10300
# rows), 16 lanes (4160: 5; 6912: 7 above), 32 lanes (8192: 4; 12288: 6;
# 11008 above), 64 lanes (16384)
MULTI_CASES = [
    [(64, (1,)), (320, (37, 129)), (1536, (300,))],
    [(3584, (16, 17)), (4160, (48,)), (8192, (77, 5))],
    [(12288, (33,)), (16384, (21,)), (1024, (256, 17, 300)), (3072, (64,))],
    [(1024, (13000,)), (2304, (10300,)), (4160, (100,))],     # 4 lanes x 6 waves; 8 lanes x 8 waves
    [(2560, (6912, 6912))],
    [(640, (50,)), (1280, (33, 9)), (1792, (70,)), (2304, (129,))],
]


@pytest.mark.parametrize("case", range(len(MULTI_CASES)))
def test_multi_shapes(case):
    spec = MULTI_CASES[case]
    groups = []
    for gi, (K, Ns) in enumerate(spec):
        seed = 1000 + 37 * case + 5 * gi + K
        Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
        _, X = workloads.small_case(seed + 99, 1, 8, K, outlier_frac=0.01)
        groups.append((Ws, X))
    print("case multi shapes %s" % (spec,), flush=True)
    out, call, name = run_multi(groups)
    assert name.startswith("fused_decode_multi_dense"), name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)
    check_same_as_single(call, out, (0, 0))


@pytest.mark.parametrize("nm", [(2, 4), (6, 8)])
def test_multi_nm_per_group_launches(nm):
    spec = [(320, (37, 129)), (4160, (48,))]
    groups = []
    for gi, (K, Ns) in enumerate(spec):
        Ws = [workloads.small_case(2000 + 7 * gi + i, 1, N, K)[0] for i, N in enumerate(Ns)]
        _, X = workloads.small_case(2050 + gi, 1, 8, K, outlier_frac=0.01)
        groups.append((Ws, X))
    print("case multi nm=%s" % (nm,), flush=True)
    out, call, name = run_multi(groups, nm)
    assert " + " in name and "multi" not in name, name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, nm, Ys, accs, xs)


def test_multi_past_the_one_launch_k():
    # a K past 16384 sends every group to its own launch
    spec = [(20480, (40,)), (256, (65,))]
    groups = []
    for gi, (K, Ns) in enumerate(spec):
        Ws = [workloads.small_case(2100 + gi + i, 1, N, K)[0] for i, N in enumerate(Ns)]
        _, X = workloads.small_case(2150 + gi, 1, 8, K, outlier_frac=0.01)
        groups.append((Ws, X))
    print("case multi K past 16384", flush=True)
    out, call, name = run_multi(groups)
    assert " + " in name, name
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)


def test_multi_zero_row_and_graph_replay():
    # an all-zero input row in one group (codes 0, scale 0, Y exactly 0);
    # the call captured in a graph and replayed gives the eager results
    import torch
    K1, K2 = 2560, 6912
    W1 = workloads.small_case(2200, 1, 700, K1)[0]
    W2 = workloads.small_case(2201, 1, 300, K2)[0]
    X1 = np.zeros((1, K1), np.float32)
    _, X2 = workloads.small_case(2202, 1, 8, K2, outlier_frac=0.01)
    groups = [([W1], X1), ([W2], X2)]
    print("case multi zero row + graph", flush=True)
    out, call, name = run_multi(groups)
    for (Ws, X), (_, Ys, accs, xs) in zip(groups, out):
        check_group(Ws, X, (0, 0), Ys, accs, xs)
    assert float(out[0][1][0].abs().max()) == 0.0
    import ternary_weight_linear_act_amd as bl
    ref = [[y.clone() for y in o[1]] for o in out]
    for o in out:
        for y in o[1]:
            y.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            bl.forward_fused_multi(call)
    torch.cuda.synchronize()
    for _ in range(3):
        for o in out:
            for y in o[1]:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, o in zip(ref, out):
            for a, b in zip(r, o[1]):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_multi_optional_outputs_and_eight_projections():
    # a group of 8 projections without accumulators or scale output beside a
    # group with both; outputs against the oracle
    import torch
    import ternary_weight_linear_act_amd as bl
    import oracle
    K1, K2 = 1024, 4160
    Ns = (16, 17, 100, 255, 256, 257, 31, 64)
    W1 = [workloads.small_case(2300 + i, 1, N, K1)[0] for i, N in enumerate(Ns)]
    W2 = [workloads.small_case(2320, 1, 333, K2)[0]]
    _, X1 = workloads.small_case(2330, 1, 8, K1, outlier_frac=0.01)
    _, X2 = workloads.small_case(2331, 1, 8, K2, outlier_frac=0.01)
    p1 = [hip_pack(W, (0, 0)) for W in W1]
    p2 = [hip_pack(W, (0, 0)) for W in W2]
    Y1 = [torch.full((1, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda") for W in W1]
    Y2 = [torch.full((1, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda") for W in W2]
    A2 = [torch.full((1, W.shape[0]), -7, dtype=torch.int32, device="cuda") for W in W2]
    xs2 = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    print("case multi 8 projections, optional outputs", flush=True)
    bl.forward_fused_multi([(to_dev(X1), [(pk, ws, W.shape[0]) for (pk, ws), W in zip(p1, W1)], Y1, None, None),
                            (to_dev(X2), [(pk, ws, W.shape[0]) for (pk, ws), W in zip(p2, W2)], Y2, A2, xs2)])
    torch.cuda.synchronize()
    assert bl.last_dispatch().startswith("fused_decode_multi_dense")
    q1, xs1_o, _ = oracle.quant_act(X1)
    for W, Y in zip(W1, Y1):
        beta, w_eff, _ = oracle.quantize_weights(W)
        acc_o, Y_o = oracle.forward(q1, xs1_o, w_eff, beta)
        check_y(Y.cpu().numpy(), Y_o, acc_o)
    check_group(W2, X2, (0, 0), Y2, A2, xs2)
