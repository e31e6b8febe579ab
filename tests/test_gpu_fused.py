"""GPU parity of the fused decode entry point (activation quantisation plus
several projections sharing the activations, one launch): bit-identical to
the two-call path and to the CPU oracle."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_forward, hip_pack, hip_quant, to_dev

pytestmark = pytest.mark.gpu


def run_fused(Ws, X, nm=(0, 0)):
    import torch
    import ternary_weight_linear_act_amd as bl
    packs = [hip_pack(W, nm) for W in Ws]
    Xd = to_dev(X)
    xs = torch.empty(X.shape[0], dtype=torch.float32, device="cuda")
    Ys, accs = bl.forward_fused(Xd, [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], nm,
                                want_acc=True, x_scale=xs)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    return packs, Ys, accs, xs, name


def check_against_oracle(Ws, X, nm, Ys, accs, xs):
    import oracle
    q, xs_o, _ = oracle.quant_act(X)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
    for W, Y, acc in zip(Ws, Ys, accs):
        beta, w_eff, _ = oracle.quantize_weights(W, *nm)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        check_y(Y.cpu().numpy(), Y_o, acc_o)


@pytest.mark.parametrize("group", [("gate", "up"), ("down",)])
def test_decode_ffn_2b_fused(group):
    d = workloads.draw("decode_ffn_2b", projs=list(group))
    Ws = [d.W[g] for g in group]
    X = d.X[(group[0], 1)]
    print("case fused decode_ffn_2b %s" % (group,), flush=True)
    _, Ys, accs, xs, name = run_fused(Ws, X)
    assert name.startswith("fused_decode") and "dense" in name, name
    check_against_oracle(Ws, X, (0, 0), Ys, accs, xs)


@pytest.mark.parametrize("group", [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)])
def test_block_3b_fused_m1(group):
    d = workloads.draw("block_3b", projs=list(group), Ms=(1,))
    Ws = [d.W[g] for g in group]
    X = d.X[(group[0], 1)]
    print("case fused block_3b %s" % (group,), flush=True)
    _, Ys, accs, xs, _ = run_fused(Ws, X)
    check_against_oracle(Ws, X, (0, 0), Ys, accs, xs)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
@pytest.mark.parametrize("K,Ns", [(64, (1,)), (320, (37, 129)), (1024, (256, 17, 300)), (4160, (48,))])
def test_fused_shapes(M, nm, K, Ns):
    rng_seed = 300 + M * 11 + K + sum(Ns)
    Ws = [workloads.small_case(rng_seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(rng_seed + 99, M, 8, K, outlier_frac=0.01)
    print("case fused M=%d K=%d Ns=%s nm=%s" % (M, K, Ns, nm), flush=True)
    _, Ys, accs, xs, _ = run_fused(Ws, X, nm)
    check_against_oracle(Ws, X, nm, Ys, accs, xs)


@pytest.mark.parametrize("M", [2, 4])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_fused_mfma_deepest_k(M, nm):
    # the largest K the 2-4-token fused kernel takes (its widest
    # configurations keep the activations partly in scratch)
    K, Ns = 16192, (300, 77)
    Ws = [workloads.small_case(800 + M + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(850 + M, M, 8, K, outlier_frac=0.01)
    print("case fused deepest K M=%d nm=%s" % (M, nm), flush=True)
    _, Ys, accs, xs, name = run_fused(Ws, X, nm)
    assert name.startswith("fused_decode_") and "dot4" not in name, name
    check_against_oracle(Ws, X, nm, Ys, accs, xs)


def test_fused_equals_two_call_path_bitwise():
    import torch
    d = workloads.draw("decode_ffn_2b", projs=["gate", "up"])
    Ws = [d.W["gate"], d.W["up"]]
    X = d.X[("gate", 1)]
    packs, Ys, accs, _, _ = run_fused(Ws, X)
    Xq, xs, rs = hip_quant(X)
    for (pk, ws), W, Y, acc in zip(packs, Ws, Ys, accs):
        Y2, acc2 = hip_forward(Xq, xs, rs, pk, ws, W.shape[0], (0, 0))
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2)
        assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


def test_fused_zero_row_and_eight_projections():
    Ws = [workloads.small_case(500 + i, 1, 16 * (i + 1) + 3, 256)[0] for i in range(8)]
    X = np.zeros((2, 256), np.float32)
    X[1] = workloads.small_case(600, 1, 8, 256)[1][0]
    _, Ys, accs, xs, _ = run_fused(Ws, X)
    check_against_oracle(Ws, X, (0, 0), Ys, accs, xs)
    assert not accs[0].cpu().numpy()[0].any()


@pytest.mark.parametrize("M", [5, 8, 9, 13, 16])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
@pytest.mark.parametrize("K,Ns", [(320, (37, 129)), (2048, (256, 300, 33)), (7936, (100,)), (11008, (70,))])
def test_fused_token_tiles(M, nm, K, Ns):
    # 5-16 tokens: tiles of 4 tokens along the grid's y, a ragged last tile,
    # several projections; against the oracle and bit for bit against the
    # two-call path
    import torch
    seed = 1300 + M * 7 + K + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 99, M, 8, K, outlier_frac=0.01)
    print("case fused tiles M=%d K=%d Ns=%s nm=%s" % (M, K, Ns, nm), flush=True)
    packs, Ys, accs, xs, name = run_fused(Ws, X, nm)
    assert name.startswith("fused_decode_") and "_mt4_tiles_" in name, name
    check_against_oracle(Ws, X, nm, Ys, accs, xs)
    Xq, xs2, rs2 = hip_quant(X)
    for (pk, ws), W, Y, acc in zip(packs, Ws, Ys, accs):
        Y2, acc2 = hip_forward(Xq, xs2, rs2, pk, ws, W.shape[0], nm)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2)
        assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


@pytest.mark.parametrize("group", [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)])
def test_block_3b_fused_m8(group):
    # the 3B block at 8 tokens, one fused launch per input group
    d = workloads.draw("block_3b", projs=list(group), Ms=(8,))
    Ws = [d.W[g] for g in group]
    X = d.X[(group[0], 8)]
    print("case fused block_3b M=8 %s" % (group,), flush=True)
    _, Ys, accs, xs, name = run_fused(Ws, X)
    assert name.startswith("fused_decode_dense"), name
    check_against_oracle(Ws, X, (0, 0), Ys, accs, xs)


def test_fused_unsupported_shapes_raise():
    import torch
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(700, 17, 64, 128)
    pk, ws = hip_pack(W, (0, 0))
    with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
        bl.forward_fused(to_dev(X), [(pk, ws, 64)])            # M = 17 > 16
    with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
        bl.forward_fused(to_dev(X[:1]), [(pk, ws, 64)] * 9)    # 9 projections
    torch.cuda.synchronize()
