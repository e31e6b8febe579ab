"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

Y_RTOL = 1e-5       # fp32 outputs: relative tolerance against the binary64 oracle


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on the CPU)"
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def hip_pack(W, nm):
    import ternary_weight_linear_act_amd as bl
    packed, ws = bl.pack_weights(to_dev(W), nm)
    return packed, ws


def hip_quant(X):
    import ternary_weight_linear_act_amd as bl
    return bl.quant_act(to_dev(X))


def hip_forward(Xq, xs, rs, packed, ws, N, nm):
    import ternary_weight_linear_act_amd as bl
    return bl.forward(Xq, xs, rs, packed, ws, N, nm, want_acc=True)


def sample_rows(M, k=16, seed=0):
    if M <= k:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=k - 2, replace=False)
    return np.unique(np.concatenate([[0, M - 1], mid]))


def check_y(Yg, Yo, acc_o):
    """Y within Y_RTOL relative of the binary64 oracle; exactly 0 where acc == 0."""
    Yg = np.asarray(Yg, np.float64)
    err = np.abs(Yg - Yo)
    bad = err > Y_RTOL * np.abs(Yo)
    assert not bad.any(), "Y: %d of %d outside %g relative (worst rel %g)" % (
        int(bad.sum()), bad.size, Y_RTOL, float((err / np.maximum(np.abs(Yo), 1e-300)).max()))
    assert np.all(Yg[acc_o == 0] == 0.0)


def full_check(W, X, nm=(0, 0), rows=None, label=""):
    """Pack + quant + forward on the GPU vs the oracle; returns the GPU tensors."""
    import torch

    import oracle
    print("case %s: M=%d N=%d K=%d nm=%s" % (label, X.shape[0], W.shape[0], W.shape[1], nm), flush=True)
    M, K = X.shape
    N = W.shape[0]
    packed, ws = hip_pack(W, nm)
    Xq, xs, rs = hip_quant(X)
    Y, acc = hip_forward(Xq, xs, rs, packed, ws, N, nm)
    torch.cuda.synchronize()

    beta, w_eff, packed_o = oracle.quantize_weights(W, *nm)
    assert np.array_equal(packed.cpu().numpy(), packed_o), "packed bytes differ"
    assert ws.cpu().numpy().view(np.uint32)[0] == np.float32(beta).view(np.uint32), "beta bits differ"
    q, xs_o, rs_o = oracle.quant_act(X)
    assert np.array_equal(Xq.cpu().numpy(), q), "Xq differs"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xs_o.view(np.uint32)), "x_scale bits differ"
    assert np.array_equal(rs.cpu().numpy(), rs_o), "row sums differ"
    if rows is None:
        rows = np.arange(M)
    if M:
        acc_o, Y_o = oracle.forward(q[rows], xs_o[rows], w_eff, beta)
        acc_g = acc.cpu().numpy()[rows]
        assert np.array_equal(acc_g, acc_o), "int32 accumulators differ in %d places" % int((acc_g != acc_o).sum())
        check_y(Y.cpu().numpy()[rows], Y_o, acc_o)
    return dict(packed=packed, ws=ws, Xq=Xq, xs=xs, rs=rs, Y=Y, acc=acc)
