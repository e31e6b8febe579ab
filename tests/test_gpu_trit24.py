"""GPU parity of the trit-packed 2:4 layout (one 6-bit code per group of 4
inputs, 12 bytes per 64 weights): the pack (bytes bit-exact with the oracle's
trit pack, beta bit-exact), the one-token kernel that looks the codes up in a
table (every lanes x strings configuration, ragged weight rows and a ragged
last string round), and the path that expands the rows to dense codes (2 to
512 tokens, and one token past K = 16384), against the CPU oracle (acc
bit-exact, Y within 1e-5) and bit-identical to the forward on the same
weights in the 2:4 values + masks layout."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, cover_rows, hip_forward, hip_pack, hip_quant, to_dev

pytestmark = pytest.mark.gpu


def trit_check(W, X, label=""):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    M, K = X.shape
    N = W.shape[0]
    print("case trit24 %s: M=%d N=%d K=%d" % (label, M, N, K), flush=True)
    packed, ws = bl.pack_weights_trit24(to_dev(W))
    Xq, xs, rs = hip_quant(X)
    Y, acc = bl.forward_trit24(Xq, xs, rs, packed, ws, N, want_acc=True)
    torch.cuda.synchronize()
    name = bl.last_dispatch()
    beta, w_eff, bytes_o = oracle.quantize_weights_trit24(W)
    assert packed.numel() == 3 * N * K // 16
    assert np.array_equal(packed.cpu().numpy(), bytes_o), "packed bytes differ"
    assert ws.cpu().numpy().view(np.uint32)[0] == np.float32(beta).view(np.uint32), "beta bits differ"
    # the same weights in the 2:4 values + masks layout
    p24, ws24 = hip_pack(W, (2, 4))
    Y24, acc24 = hip_forward(Xq, xs, rs, p24, ws24, N, (2, 4))
    torch.cuda.synchronize()
    assert torch.equal(acc, acc24) and torch.equal(Y.view(torch.int32), Y24.view(torch.int32))
    rows = cover_rows(M)
    q, xs_o, _ = oracle.quant_act(X)
    acc_o, Y_o = oracle.forward(q[rows], xs_o[rows], w_eff, beta)
    assert np.array_equal(acc.cpu().numpy()[rows], acc_o), "int32 accumulators differ"
    check_y(Y.cpu().numpy()[rows], Y_o, acc_o)
    return name


# (N, K, lanes per row, strings per lane): every configuration of the
# one-token kernel, rows not a multiple of a workgroup's, K not a multiple of
# the lanes' strings where the configuration allows it
DECODE = [(33, 64, 8, 1), (1000, 640, 8, 2), (8960, 1536, 8, 3), (70, 2048, 8, 4), (1, 2560, 8, 5),
          (500, 2624, 16, 3), (77, 4096, 16, 4), (300, 4160, 16, 5),
          (129, 5184, 32, 3), (64, 8192, 32, 4), (1536, 8960, 32, 5),
          (45, 10304, 64, 3), (203, 16384, 64, 4)]


@pytest.mark.parametrize("N,K,lpr,u", DECODE)
def test_trit24_one_token(N, K, lpr, u):
    W, X = workloads.small_case(7100 + N + K, 1, N, K, outlier_frac=0.001)
    name = trit_check(W, X, "one token")
    assert name == "trit24_decode_lpr%d_u%d" % (lpr, u), name


@pytest.mark.parametrize("M,N,K", [(2, 1000, 1536), (5, 2100, 640), (16, 8960, 1536), (17, 2560, 6912),
                                   (64, 4100, 2048), (65, 300, 192), (512, 8960, 1536), (1, 40, 16448)])
def test_trit24_expanded(M, N, K):
    W, X = workloads.small_case(7200 + M + N + K, M, N, K, outlier_frac=0.001)
    name = trit_check(W, X, "expanded")
    assert name.startswith("trit24_expand+"), name


@pytest.mark.parametrize("M", [1, 512])
@pytest.mark.parametrize("proj", ["nm24"])
def test_trit24_sparse_ffn_1p5b(proj, M):
    d = workloads.draw("sparse_ffn_1p5b", projs=[proj], Ms=(M,))
    trit_check(d.W[proj], d.X[(proj, M)], "sparse_ffn_1p5b/%s/M%d" % (proj, M))


def test_trit24_extreme_accumulators_and_zero_token():
    # W = -1 everywhere keeps inputs 0 and 1 of every group (ties to the lower
    # k); q = -128 there over the largest one-token K gives 128 * K / 2
    import torch

    import ternary_weight_linear_act_amd as bl
    N, K = 300, 16384
    W = np.full((N, K), -1.0, np.float32)
    packed, ws = bl.pack_weights_trit24(to_dev(W))
    for M, zero in ((1, None), (20, 7)):
        Xq = torch.full((M, K), -128, dtype=torch.int8, device="cuda")
        if zero is not None:
            Xq[zero] = 0
        xs = torch.ones(M, dtype=torch.float32, device="cuda")
        rs = Xq.to(torch.int32).sum(1).to(torch.int32)
        Y, acc = bl.forward_trit24(Xq, xs, rs, packed, ws, N, want_acc=True)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()
        keep = np.arange(M) != zero
        assert np.all(a[keep] == 128 * K // 2)
        if zero is not None:
            assert np.all(a[zero] == 0) and not bool(Y[zero].any())
        beta = ws.cpu().numpy()[0]
        assert np.all(Y.cpu().numpy()[keep] == np.float32(128 * K // 2) * np.float32(beta))


def test_trit24_short_workspace_and_empty_call():
    import torch

    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(7300, 8, 512, 1024)
    packed, ws = bl.pack_weights_trit24(to_dev(W))
    Xq, xs, rs = hip_quant(X)
    need = bl.forward_trit24_workspace_size(8, 512, 1024)
    assert need >= 512 * 1024 // 4
    short = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bl.BitLinearError, match="ESIZE"):
        bl.forward_trit24(Xq, xs, rs, packed, ws, 512, workspace=short)
    Y = bl.forward_trit24(Xq[:0], xs[:0], rs[:0], packed, ws, 512)
    assert Y.shape == (0, 512) and bl.last_dispatch() == "none"
