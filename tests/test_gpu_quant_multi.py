"""GPU parity of the activation quantisation of several independent inputs in
one launch (bitlinear_quant_act_multi): codes, scales and row sums of every
group bit-exact against the CPU oracle and identical to that group's own
quant_act call."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def run_multi(Xs, with_rowsum=True):
    import torch
    import ternary_weight_linear_act_amd as bl
    outs, call = [], []
    for X in Xs:
        M, K = X.shape
        Xd = to_dev(X)
        Xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
        xs = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rs = torch.full((M,), -7, dtype=torch.int32, device="cuda") if with_rowsum else None
        outs.append((Xd, Xq, xs, rs))
        call.append((Xd, Xq, xs, rs))
    bl.quant_act_multi(call)
    name = bl.last_dispatch()
    torch.cuda.synchronize()
    return outs, name


def check(Xs, outs):
    import torch
    import oracle
    import ternary_weight_linear_act_amd as bl
    for X, (Xd, Xq, xs, rs) in zip(Xs, outs):
        if X.shape[0] == 0:
            continue
        q, xs_o, rs_o = oracle.quant_act(X)
        assert np.array_equal(Xq.cpu().numpy(), q)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32))
        if rs is not None:
            assert np.array_equal(rs.cpu().numpy(), rs_o)
        Xq1, xs1, rs1 = bl.quant_act(Xd)
        torch.cuda.synchronize()
        assert torch.equal(Xq1, Xq) and torch.equal(xs1.view(torch.int32), xs.view(torch.int32))


def test_block_3b_inputs_at_8_and_64_tokens():
    # the inputs of the 3B block's q/k/v, gate/up and down groups
    for M in (8, 64):
        d = workloads.draw("block_3b", Ms=(M,))
        Xs = [d.X[("q", M)], d.X[("gate", M)], d.X[("down", M)]]
        print("case quant multi block_3b M=%d" % M, flush=True)
        outs, name = run_multi(Xs)
        assert name == "quant_act_multi", name
        check(Xs, outs)


@pytest.mark.parametrize("spec", [
    [(1, 64), (3, 320), (17, 1024)],                 # 256 threads, 1 float4 per thread
    [(2, 4096), (5, 11008), (1, 16384)],             # 1024 threads, up to 4
    [(300, 2560), (300, 2048)],                      # past 512 rows: 256 threads, up to 8 (K <= 8192)
    [(0, 2048), (4, 6912), (0, 128), (9, 64)],       # empty groups
    [(1, 64)] * 8,                                   # eight groups
])
def test_quant_multi_shapes(spec):
    Xs = [workloads.small_case(3000 + 17 * i + K + M, M, 8, K, outlier_frac=0.01)[1] for i, (M, K) in
          enumerate(spec)]
    print("case quant multi %s" % (spec,), flush=True)
    outs, name = run_multi(Xs)
    assert name == "quant_act_multi", name
    check(Xs, outs)


def test_quant_multi_zero_and_tiny_rows_without_rowsum():
    X1 = np.zeros((3, 2048), np.float32)
    X2 = np.full((2, 4096), 2.0 ** -120, np.float32)
    X2[1, ::7] = -(2.0 ** -110)
    Xs = [X1, X2]
    print("case quant multi zero and tiny rows", flush=True)
    outs, name = run_multi(Xs, with_rowsum=False)
    check(Xs, outs)
    assert float(outs[0][2].abs().max()) == 0.0


def test_quant_multi_per_group_past_the_registers():
    # 600 rows of K = 12288 do not fit 256 threads x 8 float4: one launch per group
    Xs = [workloads.small_case(3100, 600, 8, 12288, outlier_frac=0.01)[1],
          workloads.small_case(3101, 3, 8, 256)[1]]
    print("case quant multi per group", flush=True)
    outs, name = run_multi(Xs)
    assert name == "quant_act per group", name
    check(Xs, outs)
