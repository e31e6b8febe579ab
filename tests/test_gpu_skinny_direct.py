"""GPU parity of the skinny MFMA forward that reads the packed weights straight
into the MFMA operand (dense weights at 5-64 tokens, the shapes where it
measured faster than the staged kernel): every rule of its dispatch at its
edges, with ragged weight rows (a partial last column block), against the
CPU oracle (acc bit-exact, Y within 1e-5) and bit-identical to the forward
of each projection alone.  Next to each rule, a shape just outside it takes
the staged kernel.  Wide projections at 9-64 tokens take the form with
several token tiles per workgroup (tested on its own); grouped calls past
the skinny tiles' workgroup limit take the few-token GEMM's grouped launch
where its rule holds."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, cover_rows, direct_tiles, full_check, hip_forward, hip_pack, hip_quant, skinny_direct

pytestmark = pytest.mark.gpu


# (M, N, K): each rule at its smallest and largest K and token count
SINGLE = [
    (5, 8200, 512), (8, 8200, 2048), (6, 8192, 1024),          # 5-8 tokens, K <= 2048, >= 8192 rows
    (5, 8200, 2112), (8, 8200, 2560),                          # 5-8 tokens, K 2112-2560
    (5, 300, 8256), (8, 300, 12288), (7, 2048, 11008),         # 5-8 tokens, deep K
]


@pytest.mark.parametrize("M,N,K", SINGLE)
def test_direct_single(M, N, K):
    import ternary_weight_linear_act_amd as bl
    assert skinny_direct(M, K, N)
    W, X = workloads.small_case(5100 + M + K + N, M, N, K, outlier_frac=0.001)
    full_check(W, X, (0, 0), label="skinny-direct")
    name = bl.last_dispatch()
    assert name.startswith("skinny_direct_dense_"), name


@pytest.mark.parametrize("M,N,K", [(4, 8200, 2048), (8, 8191, 2048), (8, 8200, 448), (17, 2500, 2048),
                                   (8, 8200, 2624), (8, 300, 8192), (8, 300, 12352), (12, 6900, 2048)])
def test_outside_rules_take_the_staged_kernel(M, N, K):
    import ternary_weight_linear_act_amd as bl
    assert not skinny_direct(M, K, N) and not direct_tiles(M, K, N)
    W, X = workloads.small_case(5200 + M + K + N, M, N, K)
    full_check(W, X, (0, 0), rows=cover_rows(M), label="skinny-direct-outside")
    assert not bl.last_dispatch().startswith("skinny_direct"), bl.last_dispatch()


@pytest.mark.parametrize("nm", [(2, 4), (6, 8)])
def test_nm_patterns_keep_their_kernels(nm):
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(5300, 8, 8200, 2048)
    full_check(W, X, nm, label="skinny-direct-nm")
    assert not bl.last_dispatch().startswith("skinny_direct"), bl.last_dispatch()


@pytest.mark.parametrize("M", [5, 8, 16, 17, 33, 64])
@pytest.mark.parametrize("K,Ns", [(512, (300, 17)), (2048, (4100, 4100)), (2048, (2048, 2048)),
                                  (2048, (2048, 256, 256))])
def test_direct_grouped(M, K, Ns):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    seed = 5400 + M + K + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 99, M, 8, K, outlier_frac=0.01)
    print("case direct grouped M=%d K=%d Ns=%s" % (M, K, Ns), flush=True)
    packs = [hip_pack(W, (0, 0)) for W in Ws]
    Xq, xs, rs = hip_quant(X)
    projs = [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)]
    tiles = direct_tiles(M, K, sum(Ns))
    past_skinny = M > 16 and sum(-(-N // 16) for N in Ns) * -(-M // 16) > 1024
    gemm = M > 16 and len(Ns) > 1 and all((K <= 4096 or N >= 8192) and -(-M // 32) * -(-N // 32) >= 256 for N in Ns)
    if not tiles and past_skinny and not gemm:
        # past 16 tokens the skinny tiles take at most 1024 workgroups, and
        # the grouped GEMM wants a tile per compute unit in every projection
        with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
            bl.forward_grouped(Xq, xs, rs, projs)
        return
    Ys, accs = bl.forward_grouped(Xq, xs, rs, projs, want_acc=True)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    if tiles:
        assert name == tiles + "_grouped", name
    elif past_skinny:
        assert name == "gemm_dense_dma_32x32_grouped", name
    elif skinny_direct(M, K, sum(Ns), len(Ns)):
        assert name.startswith("skinny_direct_dense_") and name.endswith("_grouped"), name
    else:
        assert not name.startswith("skinny_direct"), name
    rows = cover_rows(M)
    q, xs_o, _ = oracle.quant_act(X[rows])
    for (pk, ws), W, Y, acc in zip(packs, Ws, Ys, accs):
        Y2, acc2 = hip_forward(Xq, xs, rs, pk, ws, W.shape[0], (0, 0))
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2) and torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
        beta, w_eff, _ = oracle.quantize_weights(W, 0, 0)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy()[rows], acc_o)
        check_y(Y.cpu().numpy()[rows], Y_o, acc_o)


def test_extreme_accumulators_and_zero_rows():
    # q = -128 against t = -1 over the whole of a deep K, and an all-zero token
    import torch

    import ternary_weight_linear_act_amd as bl
    M, N, K = 8, 8200, 2048
    W = np.full((N, K), -1.0, np.float32)
    X = np.full((M, K), -1.0, np.float32)
    X[3] = 0.0
    packed, ws = hip_pack(W, (0, 0))
    Xq = torch.full((M, K), -128, dtype=torch.int8, device="cuda")
    Xq[3] = 0
    xs = torch.ones(M, dtype=torch.float32, device="cuda")
    rs = Xq.to(torch.int32).sum(1).to(torch.int32)
    Y, acc = hip_forward(Xq, xs, rs, packed, ws, N, (0, 0))
    torch.cuda.synchronize()
    assert bl.last_dispatch().startswith("skinny_direct_dense_"), bl.last_dispatch()
    a = acc.cpu().numpy()
    assert np.all(a[3] == 0) and np.all(np.delete(a, 3, axis=0) == 128 * K)
    assert not bool(Y[3].any())
