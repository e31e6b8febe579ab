"""GPU parity of the H-BitLinear activation path (the BitNet v2 summary: the
activations entering a projection are Hadamard-transformed online, then
quantised to 4 bits), compared with the CPU oracle:
- bitlinear_quant_act_h4: codes, row sums and x_scale bit-exact, for block
  sizes 1 to 8192 and rows of one or several LDS chunks (K > 8192, with a
  partial last chunk);
- a tiny row (one-hot 2^-126, where 7/g would overflow) and a zero row;
- quant_act_h4 then bitlinear_forward, dense and 2:4: acc bit-exact, Y
  within 1e-5 relative.

Inputs are seeded N(0,1) activations with 1% outliers x20."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_pack, to_dev

pytestmark = pytest.mark.gpu


def rows(seed, M, K):
    X = workloads.activations(np.random.default_rng(seed), M, K, 0.01)
    if M >= 3:
        X[1] = 0.0
        X[2] = 0.0
        X[2, 9] = np.float32(2.0 ** -126)
    return X


def h4_kernel(K, B):
    """The quantiser the library picks: one block per wave in registers for
    64 <= B <= 1024 with at most 16 waves of 16 / (B / 64) blocks, else the
    LDS form."""
    if 64 <= B <= 1024 and K // B <= 16 * (16 // (B // 64)):
        return "quant_act_h4_wave"
    return "quant_act_h4"


@pytest.mark.parametrize("M,K,B", [(1, 64, 64), (3, 2560, 512), (5, 6912, 256), (2, 16384, 8192),
                                   (4, 11008, 256), (7, 512, 1), (3, 512, 2), (3, 512, 4), (2, 1024, 8),
                                   (2, 1024, 16), (3, 4096, 4096), (2, 24576, 8192), (3, 2048, 128),
                                   (3, 16384, 1024), (3, 17408, 1024), (3, 16384, 64), (3, 16448, 64),
                                   (4, 1024, 1024), (3, 8192, 512), (5, 8256, 64), (300, 6912, 256)])
def test_quant_act_h4(M, K, B):
    # both forms: the wave form at B = 64 .. 1024 up to its largest row (16
    # waves of 16 / (B / 64) blocks) and one block past it (the LDS form),
    # one-wave rows, a ragged last wave, many rows
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    X = rows(700 + K + B, M, K)
    print("case quant_act_h4 M=%d K=%d B=%d" % (M, K, B), flush=True)
    q, xs, rs = bl.quant_act_h4(to_dev(X), B)
    assert bl.last_dispatch() == h4_kernel(K, B), bl.last_dispatch()
    torch.cuda.synchronize()
    q_o, xs_o, rs_o = oracle.quant_act_h4(X, B)
    assert np.array_equal(q.cpu().numpy(), q_o)
    assert np.array_equal(rs.cpu().numpy(), rs_o)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))


@pytest.mark.parametrize("M,N,K,B", [(1, 2560, 6912, 256), (1, 2048, 2048, 2048), (64, 1000, 2560, 512),
                                     (512, 2048, 6912, 256)])
@pytest.mark.parametrize("nm", [(0, 0), (2, 4)])
def test_h_bitlinear_forward(M, N, K, B, nm):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(750 + M + K, M, N, K, outlier_frac=0.01)
    print("case h-bitlinear M=%d N=%d K=%d B=%d nm=%s" % (M, N, K, B, nm), flush=True)
    pk, ws = hip_pack(W, nm)
    Xq, xs, rs = bl.quant_act_h4(to_dev(X), B)
    Y, acc = bl.forward(Xq, xs, rs, pk, ws, N, nm, want_acc=True)
    torch.cuda.synchronize()
    q_o, xs_o, _ = oracle.quant_act_h4(X, B)
    beta, w_eff, _ = oracle.quantize_weights(W, *nm)
    sel = np.unique(np.linspace(0, M - 1, min(M, 16)).astype(int))
    acc_o, Y_o = oracle.forward(q_o[sel], xs_o[sel], w_eff, beta)
    assert np.array_equal(acc.cpu().numpy()[sel], acc_o)
    check_y(Y.cpu().numpy()[sel], Y_o, acc_o)
