"""GPU parity of the one-token decode kernel on packed int8 dot products
(M = 1, K <= 16384), plain and with the activation quantisation fused in.

The kernel picks 8, 16, 32 or 64 lanes per weight row from K (at most 5
chunks of 64 weights per lane, 7 with the quantisation fused in); the K
values below cover every lane count of both rules at its largest and
smallest chunk count, with ragged N (rows past the last workgroup's first
row).  Past K = 16384 the
calls fall back to the MFMA kernels.  Everything is checked against the CPU
oracle: int32 accumulators, x_scale bits and row sums bit-exact, Y within
1e-5 relative."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, full_check, hip_pack, to_dev

pytestmark = pytest.mark.gpu

K_CASES = [64, 2560, 2624, 3584, 3648, 5120, 5184, 7168, 7232, 10240, 10304, 14336, 14400, 16384]


def expected_config(K, fused):
    """(lanes per row, chunks per lane) the host picks for K."""
    C, umax, lpr = K // 64, (7 if fused else 5), 8
    while lpr < 64 and -(-C // lpr) > umax:
        lpr *= 2
    return lpr, -(-C // lpr)
NM_CASES = [(0, 0), (2, 4), (6, 8)]


@pytest.mark.parametrize("K", K_CASES)
@pytest.mark.parametrize("nm", NM_CASES)
def test_forward_m1(K, nm):
    import ternary_weight_linear_act_amd as bl
    N = 37 if K > 4096 else 301
    W, X = workloads.small_case(4000 + K + N, 1, N, K, outlier_frac=0.01)
    full_check(W, X, nm, label="dot4 forward")
    name = bl.last_dispatch()
    assert name.startswith("decode_dot4_") and ("_lpr%d_u%d_" % expected_config(K, False)) in name, name


def fused_vs_oracle(Ws, X, nm):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    packs = [hip_pack(W, nm) for W in Ws]
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    Ys, accs = bl.forward_fused(to_dev(X), [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)], nm,
                                want_acc=True, x_scale=xs)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    q, xs_o, _ = oracle.quant_act(X)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
    for W, Y, acc in zip(Ws, Ys, accs):
        beta, w_eff, _ = oracle.quantize_weights(W, *nm)
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        check_y(Y.cpu().numpy(), Y_o, acc_o)
    return name


@pytest.mark.parametrize("K", K_CASES)
@pytest.mark.parametrize("nm", NM_CASES)
def test_fused_m1(K, nm):
    Ns = (29, 70, 5) if K > 4096 else (130, 257, 3)
    Ws = [workloads.small_case(5000 + K + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(5100 + K, 1, 8, K, outlier_frac=0.01)
    print("case dot4 fused K=%d Ns=%s nm=%s" % (K, Ns, nm), flush=True)
    name = fused_vs_oracle(Ws, X, nm)
    assert name.startswith("fused_decode_dot4_") and ("_lpr%d_u%d_p3" % expected_config(K, True)) in name, name


@pytest.mark.parametrize("nm", NM_CASES)
@pytest.mark.parametrize("K", [1024, 3584])
def test_fused_m1_eight_waves(K, nm):
    # more than 320 four-wave workgroups at 8 lanes per row: 8 waves, 64 rows
    Ns = (9000, 2000, 70)
    Ws = [workloads.small_case(5400 + K + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(5500 + K, 1, 8, K, outlier_frac=0.01)
    print("case dot4 fused 8 waves K=%d nm=%s" % (K, nm), flush=True)
    name = fused_vs_oracle(Ws, X, nm)
    assert name.startswith("fused_decode_dot4_") and "_lpr8_" in name and name.endswith("_p3_w8"), name


@pytest.mark.parametrize("nm", NM_CASES)
def test_fused_m1_eight_projections(nm):
    # the most projections one launch takes, of uneven sizes (one a single row)
    Ns = (1, 37, 300, 64, 513, 7, 129, 2000)
    K = 1536
    Ws = [workloads.small_case(5600 + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(5700, 1, 8, K, outlier_frac=0.01)
    print("case dot4 fused 8 projections nm=%s" % (nm,), flush=True)
    name = fused_vs_oracle(Ws, X, nm)
    assert name.startswith("fused_decode_dot4_") and name.endswith("_p8"), name


@pytest.mark.parametrize("nm", NM_CASES)
def test_zero_row_m1(nm):
    import torch

    import ternary_weight_linear_act_amd as bl
    W, _ = workloads.small_case(5200, 1, 65, 1024)
    X = np.zeros((1, 1024), np.float32)
    r = full_check(W, X, nm, label="dot4 zero row")
    assert bl.last_dispatch().startswith("decode_dot4_")
    assert not r["acc"].cpu().numpy().any() and not torch.any(r["Y"] != 0)
    name = fused_vs_oracle([W], X, nm)
    assert name.startswith("fused_decode_dot4_")


def test_large_k_falls_back_to_mfma():
    import ternary_weight_linear_act_amd as bl
    K = 16448
    W, X = workloads.small_case(5300, 1, 40, K, outlier_frac=0.01)
    full_check(W, X, (0, 0), label="dot4 fallback")
    assert not bl.last_dispatch().startswith("decode_dot4"), bl.last_dispatch()
    name = fused_vs_oracle([W], X, (0, 0))
    assert name.startswith("fused_decode") and "dot4" not in name, name
