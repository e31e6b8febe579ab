"""GPU parity of the grouped forward (several projections sharing one
quantised input, one launch): bit-identical to bitlinear_forward per
projection, and equal to the CPU oracle (acc bit-exact, Y within 1e-5)."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, cover_rows, direct_tiles, hip_forward, hip_pack, hip_quant, skinny_direct

pytestmark = pytest.mark.gpu


def run_grouped(Ws, X, nm):
    import torch

    import ternary_weight_linear_act_amd as bl
    packs = [hip_pack(W, nm) for W in Ws]
    Xq, xs, rs = hip_quant(X)
    Ys, accs = bl.forward_grouped(Xq, xs, rs, [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], nm,
                                  want_acc=True)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    return packs, (Xq, xs, rs), Ys, accs, name


def check(Ws, X, nm, packs, xq, Ys, accs):
    import torch

    import oracle
    rows = cover_rows(X.shape[0])
    q, xs_o, _ = oracle.quant_act(X[rows])
    for (pk, ws), W, Y, acc in zip(packs, Ws, Ys, accs):
        Y2, acc2 = hip_forward(*xq, pk, ws, W.shape[0], nm)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2), "grouped and single forward differ"
        assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
        beta, w_eff, _ = oracle.quantize_weights(W, *nm)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy()[rows], acc_o)
        check_y(Y.cpu().numpy()[rows], Y_o, acc_o)


@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 17, 40, 64])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
@pytest.mark.parametrize("K,Ns", [(256, (37, 129)), (2048, (256, 300, 33)), (6912, (100, 64))])
def test_grouped_shapes(M, nm, K, Ns):
    seed = 4400 + M * 3 + K + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 77, M, 8, K, outlier_frac=0.01)
    print("case grouped M=%d K=%d Ns=%s nm=%s" % (M, K, Ns, nm), flush=True)
    if K == 6912 and M > 8:
        # 16 staged token rows of K = 6912 leave no skinny configuration
        # within the LDS: the call is refused and launches nothing
        import ternary_weight_linear_act_amd as bl
        with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
            run_grouped(Ws, X, nm)
        return
    packs, xq, Ys, accs, name = run_grouped(Ws, X, nm)
    if M == 1:
        assert name.startswith("decode_dot4") and name.endswith("_p%d" % len(Ns)), name
    elif skinny_direct(M, K, sum(Ns), len(Ns), nm):
        assert name.startswith("skinny_direct_dense_") and name.endswith("_grouped"), name
    else:
        assert name.startswith("skinny_mfma") and name.endswith("_grouped"), name
    check(Ws, X, nm, packs, xq, Ys, accs)


@pytest.mark.parametrize("M", [8])
def test_block_3b_gate_up_grouped(M):
    d = workloads.draw("block_3b", projs=["gate", "up"], Ms=(M,))
    Ws = [d.W["gate"], d.W["up"]]
    X = d.X[("gate", M)]
    print("case grouped block_3b gate+up M=%d" % M, flush=True)
    packs, xq, Ys, accs, name = run_grouped(Ws, X, (0, 0))
    assert name.endswith("_grouped"), name
    check(Ws, X, (0, 0), packs, xq, Ys, accs)


@pytest.mark.parametrize("M,nm", [(40, (0, 0)), (64, (0, 0)), (64, (2, 4)), (64, (6, 8))])
def test_block_3b_qkv_grouped_many_workgroups(M, nm):
    # q, k, v of the 3B block past 16 tokens (2560 rows in all): dense on the
    # direct-load token-tile kernel; N:M on the skinny kernel's 160 rows of 16
    # in 3 or 4 token tiles, 480 or 640 workgroups (a grouped call of several
    # projections takes up to 1024)
    d = workloads.draw("block_3b", projs=["q", "k", "v"], Ms=(64,))
    Ws = [d.W["q"], d.W["k"], d.W["v"]]
    X = d.X[("q", 64)][:M]
    print("case grouped block_3b q+k+v M=%d nm=%s" % (M, nm), flush=True)
    packs, xq, Ys, accs, name = run_grouped(Ws, X, nm)
    if nm == (0, 0):
        assert name == direct_tiles(M, 2048, 2560) + "_grouped", name
    else:
        assert name.startswith("skinny_mfma") and name.endswith("_grouped"), name
    check(Ws, X, nm, packs, xq, Ys, accs)


def test_grouped_unsupported_raises():
    import torch

    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(4500, 64, 11008, 2048)
    pk, ws = hip_pack(W, (0, 0))
    Xq, xs, rs = hip_quant(X)
    # one projection of 2080 rows over K = 3136 (49 chunks, past the
    # token-tile kernel): 520 skinny workgroups at 64 tokens are too many for
    # a single projection (512), and the grouped GEMM takes two or more
    W2, X2 = workloads.small_case(4501, 64, 2080, 3136)
    pk2, ws2 = hip_pack(W2, (0, 0))
    Xq2, xs2, rs2 = hip_quant(X2)
    with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
        bl.forward_grouped(Xq2, xs2, rs2, [(pk2, ws2, 2080)])
    # a wide projection beside one of too few GEMM tiles (3000 rows: 188 of
    # 32 x 32 at 64 tokens, below one per compute unit); 14008 rows in all is
    # outside the token-tile kernel's rules at 33-64 tokens
    W4, _ = workloads.small_case(4503, 1, 3000, 2048)
    pk4, ws4 = hip_pack(W4, (0, 0))
    with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
        bl.forward_grouped(Xq, xs, rs, [(pk, ws, 11008), (pk4, ws4, 3000)])
    # deep K over few rows: neither the skinny tiles (LDS) nor the grouped GEMM
    W3, X3 = workloads.small_case(4502, 64, 2048, 11008)
    pk3, ws3 = hip_pack(W3, (0, 0))
    Xq3, xs3, rs3 = hip_quant(X3)
    with pytest.raises(bl.BitLinearError, match="EUNSUPPORTED"):
        bl.forward_grouped(Xq3, xs3, rs3, [(pk3, ws3, 2048), (pk3, ws3, 2048)])
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,Ns", [(64, 2560, (6912, 6912)), (17, 3136, (8192, 8300)), (33, 3200, (8200, 12000, 8192)),
                                    (48, 4096, (8200, 8200)), (64, 6144, (8192, 8200))])
def test_grouped_gemm(M, K, Ns):
    # past the skinny kernel's workgroup limit and outside the token-tile
    # kernel's rules: one launch of the few-token GEMM's 32 x 32 tiles for all
    # projections (ragged weight rows, a ragged last token tile)
    assert direct_tiles(M, K, sum(Ns)) is None
    seed = 4600 + M + K + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 77, M, 8, K, outlier_frac=0.01)
    print("case grouped GEMM M=%d K=%d Ns=%s" % (M, K, Ns), flush=True)
    packs, xq, Ys, accs, name = run_grouped(Ws, X, (0, 0))
    assert name == "gemm_dense_dma_32x32_grouped", name
    check(Ws, X, (0, 0), packs, xq, Ys, accs)


@pytest.mark.parametrize("M", [16, 32, 64])
def test_block_3b_gate_up_grouped_full_size(M):
    # gate + up of the 3B block (2 x 11008 rows, K = 2048) in one launch of the
    # direct-load kernel with several token tiles per workgroup
    d = workloads.draw("block_3b", projs=["gate", "up"], Ms=(64,))
    Ws = [d.W["gate"], d.W["up"]]
    X = d.X[("gate", 64)][:M]
    print("case grouped block_3b gate+up M=%d" % M, flush=True)
    packs, xq, Ys, accs, name = run_grouped(Ws, X, (0, 0))
    assert name == direct_tiles(M, 2048, 22016) + "_grouped", name
    check(Ws, X, (0, 0), packs, xq, Ys, accs)
