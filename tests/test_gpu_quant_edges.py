"""GPU parity of activation quantisation on rows of tiny magnitude, through
every kernel that quantises: bitlinear_quant_act, the fused one-token decode
kernel (M = 1) and the fused MFMA decode kernel (M = 2-4).

A row with max|x| below 2^-100 is scaled by 2^100 before s = 127/max|x| is
formed (below 127/FLT_MAX that quotient overflows).  Rows here: the pinned
hand example at 2^-125 tiled along K (s would overflow), values of magnitude
[1, 2) times 2^-124 with zeros, the same at 2^-101 (scaled, s finite), and
an ordinary row.  q, x_scale, row sums and the int32 accumulators are
compared bit for bit with the oracle; Y where it is a normal float."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_forward, hip_pack, hip_quant, to_dev

pytestmark = pytest.mark.gpu

K = 1024


def tiny_rows():
    rng = np.random.default_rng(77)
    hand = np.tile(np.array([2.0 ** -125, -(2.0 ** -125), 0.0, 2.0 ** -127]), K // 4)
    mag = rng.uniform(1.0, 2.0, K) * rng.choice([-1.0, 1.0], K)
    mag[::13] = 0.0
    rows = [hand, mag * 2.0 ** -124, mag * 2.0 ** -101, workloads.small_case(78, 1, 8, K)[1][0]]
    return np.array(rows, np.float32)


def oracle_ref(X, W):
    import oracle
    q, xs, rs = oracle.quant_act(X)
    beta, w_eff, _ = oracle.quantize_weights(W)
    acc, Y = oracle.forward(q, xs, w_eff, beta)
    return q, xs, rs, acc, Y


def test_quant_act_tiny_rows():
    import torch
    X = tiny_rows()
    q, xs, rs = hip_quant(X)
    torch.cuda.synchronize()
    import oracle
    q_o, xs_o, rs_o = oracle.quant_act(X)
    assert q_o[0, :4].tolist() == [127, -127, 0, 32]
    assert np.array_equal(q.cpu().numpy(), q_o)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
    assert np.array_equal(rs.cpu().numpy(), rs_o)


@pytest.mark.parametrize("row", [0, 1, 2, 3])
def test_one_token_paths_tiny_rows(row):
    import torch

    import ternary_weight_linear_act_amd as bl
    X = tiny_rows()[row:row + 1]
    W = workloads.small_case(79, 1, 200, K)[0]
    q_o, xs_o, rs_o, acc_o, Y_o = oracle_ref(X, W)
    pk, ws = hip_pack(W, (0, 0))
    Xq, xs, rs = hip_quant(X)
    Y, acc = hip_forward(Xq, xs, rs, pk, ws, 200, (0, 0))
    name = bl.last_dispatch()
    xs_f = torch.empty(1, dtype=torch.float32, device="cuda")
    Ys, accs = bl.forward_fused(to_dev(X), [(pk, ws, 200)], want_acc=True, x_scale=xs_f)
    fname = bl.last_dispatch()
    torch.cuda.synchronize()
    print("case tiny row %d: %s, %s" % (row, name, fname), flush=True)
    assert name.startswith("decode_dot4_") and fname.startswith("fused_decode_dot4_")
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert np.array_equal(accs[0].cpu().numpy(), acc_o)
    assert np.array_equal(xs_f.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
    if row >= 2:                                   # x_scale normal: Y normal too
        check_y(Y.cpu().numpy(), Y_o, acc_o)
        check_y(Ys[0].cpu().numpy(), Y_o, acc_o)


@pytest.mark.parametrize("M", [2, 4])
def test_fused_mfma_tiny_rows(M):
    import torch

    import ternary_weight_linear_act_amd as bl
    X = tiny_rows()[:M] if M == 4 else tiny_rows()[[0, 2]]
    W = workloads.small_case(80, 1, 96, K)[0]
    q_o, xs_o, rs_o, acc_o, Y_o = oracle_ref(X, W)
    pk, ws = hip_pack(W, (0, 0))
    xs_f = torch.empty(M, dtype=torch.float32, device="cuda")
    Ys, accs = bl.forward_fused(to_dev(X), [(pk, ws, 96)], want_acc=True, x_scale=xs_f)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    print("case fused tiny rows M=%d: %s" % (M, name), flush=True)
    assert name.startswith("fused_decode_") and "dot4" not in name
    assert np.array_equal(accs[0].cpu().numpy(), acc_o)
    assert np.array_equal(xs_f.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
