"""GPU parity of BitNet a4.8's hybrid activations: bitlinear_quant_act_a48
bit-exact against the oracle (codes of both parts, scales, row sums), with
many ties at the outlier threshold, tiny and zero rows, T = 0 and T = K; and
the whole path (quant_act_a48, bitlinear_forward on the 2M rows,
bitlinear_combine_a48): accumulators bit-exact, Y within 1e-5 relative to
the magnitude of its two parts."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import hip_pack, to_dev

pytestmark = pytest.mark.gpu


def gpu_a48(X, T):
    import torch

    import ternary_weight_linear_act_amd as bl
    Xq, xs, rs = bl.quant_act_a48(to_dev(X), T)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), xs.cpu().numpy(), rs.cpu().numpy()


def check_quant(X, T):
    import oracle
    q, xs, rs = gpu_a48(X, T)
    qo, xso, rso, _ = oracle.quant_act_a48(X, T)
    assert np.array_equal(q, qo), "codes differ in %d places" % int((q != qo).sum())
    assert np.array_equal(xs.view(np.uint32), xso.view(np.uint32)), "scales differ"
    assert np.array_equal(rs, rso), "row sums differ"


@pytest.mark.parametrize("K", [64, 320, 2560, 4096, 6912, 11008, 16384])
def test_quant_a48_shapes(K):
    rng = np.random.default_rng(6000 + K)
    X = workloads.activations(rng, 37, K, 0.01)
    for T in sorted({0, 1, 3, K // 100, K // 10, K - 1, K}):
        print("case a48 quant K=%d T=%d" % (K, T), flush=True)
        check_quant(X, T)


@pytest.mark.parametrize("K", [256, 2560, 6912])
def test_quant_a48_ties(K):
    # values from a handful of magnitudes: the threshold falls inside a run of
    # equal keys, which must be split in k order
    rng = np.random.default_rng(6100 + K)
    X = (rng.integers(-4, 5, size=(24, K)) * 0.375).astype(np.float32)
    for T in (1, 5, K // 7, K // 3, K // 2):
        print("case a48 ties K=%d T=%d" % (K, T), flush=True)
        check_quant(X, T)


def test_quant_a48_tiny_and_zero_rows():
    X = np.zeros((4, 512), np.float32)
    X[1, 7] = 2.0 ** -126
    X[1, 300] = -(2.0 ** -127)
    X[2] = workloads.activations(np.random.default_rng(6200), 1, 512)[0] * np.float32(2.0 ** -110)
    X[3, :5] = 1.0
    for T in (0, 1, 2, 5, 6, 512):
        print("case a48 tiny T=%d" % T, flush=True)
        check_quant(X, T)


@pytest.mark.parametrize("M,N,K,T", [(1, 2560, 6912, 69), (1, 6912, 2560, 26), (7, 300, 1024, 10),
                                     (64, 2048, 2048, 20), (512, 1536, 2560, 128)])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (6, 8)])
def test_a48_forward(M, N, K, T, nm):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(6300 + M + K, M, N, K, outlier_frac=0.001)
    print("case a48 forward M=%d N=%d K=%d T=%d nm=%s" % (M, N, K, T, nm), flush=True)
    pk, ws = hip_pack(W, nm)
    Xq, xs, rs = bl.quant_act_a48(to_dev(X), T)
    Y2, acc2 = bl.forward(Xq, xs, rs, pk, ws, N, nm, want_acc=True)
    Y = bl.combine_a48(Y2)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 24)).astype(int))
    q2, xs2, _, _ = oracle.quant_act_a48(X[rows], T)
    beta, w_eff, _ = oracle.quantize_weights(W, *nm)
    acc_o, Y_o, Yp_o = oracle.forward_a48(q2, xs2, w_eff, beta)
    rows2 = np.stack([2 * rows, 2 * rows + 1], 1).reshape(-1)
    assert np.array_equal(acc2.cpu().numpy()[rows2], acc_o)
    Yg = Y.cpu().numpy().astype(np.float64)[rows]
    mag = np.abs(Yp_o[0::2]) + np.abs(Yp_o[1::2])
    err = np.abs(Yg - Y_o)
    assert np.all(err <= 1e-5 * mag), float((err / np.maximum(mag, 1e-300)).max())
    assert np.all(Yg[(acc_o[0::2] == 0) & (acc_o[1::2] == 0)] == 0.0)
