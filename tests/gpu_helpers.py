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


def cover_rows(M):
    """Rows compared at full size: every row up to 64 tokens; beyond, rows
    chosen so that every 32-row block of the output (and so every tile of any
    kernel here: 32 to 256 rows, the XCD regions of the tile grid) holds at
    least one, all 32 residues mod 32 (the row positions inside an MFMA
    fragment) occur, and the first and last rows are included."""
    if M <= 64:
        return np.arange(M)
    blocks = -(-M // 32)
    per = -(-32 // blocks)                 # rows per block so that the residues cover 0..31
    rows = [0, M - 1]
    for i in range(blocks):
        for j in range(per):
            r = 32 * i + (i * per + j) % 32
            if r < M:
                rows.append(r)
    # a ragged last block can drop residues: take those from the first block
    rows += [r for r in range(32) if r not in {x % 32 for x in rows}]
    return np.unique(np.array(rows))


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


def skinny_direct(M, K, rows, nproj=1, nm=(0, 0)):
    """Dense weights at 5-64 tokens where the library reads the weights
    straight into the MFMA operand (the shapes where that measured faster)."""
    C = K // 64
    if nm != (0, 0):
        return False
    wide = rows >= 8192
    return ((5 <= M <= 8 and 8 <= C <= 32 and wide)
            or (5 <= M <= 8 and 32 < C <= 40 and wide) or (5 <= M <= 8 and 128 < C <= 192)
            or (17 <= M <= 64 and nproj >= 2 and 8 <= C <= 32 and not direct_tiles(M, K, rows)))


def direct_tiles(M, K, rows, nm=(0, 0)):
    """Dense weights at 9-64 tokens over at least 6912 weight rows (all
    projections of a call together), 2560 from 17 tokens or 2048 from 33, K of 4 to 48
    chunks of 64: the direct-load kernel with several 16-token tiles per
    workgroup.  Its dispatch name (without the "_grouped" of a grouped call),
    or None."""
    C = K // 64
    if nm != (0, 0) or not (9 <= M <= 64) or not (4 <= C <= 48) or rows < 2048:
        return None
    s = 2 if C <= 32 else 3
    if rows < 6912:
        if M < (33 if rows < 2560 else 17):
            return None
        tt, rg = 1, 2
    elif M <= 16:
        tt, rg = 1, 2
    elif M <= 32:
        tt, rg = (1, 4) if rows >= 13824 else (1, 2)
    elif rows < 13824:
        tt, rg = 1, 4
    elif rows >= 16384 and C <= 32:
        tt, rg = 2, 6
    else:
        return None
    return "skinny_direct_tiles_dense_t%d_rg%d_s%d" % (tt, rg, s)


def direct_tiles_split(M, K, N, nm=(0, 0)):
    """One dense projection at 9-64 tokens with K of 49 to 384 chunks of 64 and
    1024 to 4096 weight rows (2560 past 32 tokens): the token-tile kernel with
    K split into ceil(C / 48) parts over the workgroups, where the staged
    skinny kernel does not take the shape first.  Its dispatch name, or None."""
    C = K // 64
    if nm != (0, 0) or not (9 <= M <= 64) or not (48 < C <= 384) or not (1024 <= N <= (4096 if M <= 32 else 2560)):
        return None
    tt, rg = (1, 2) if M <= 32 else (2, 4)
    return "skinny_direct_tiles_dense_t%d_rg%d_s3_splitk%d" % (tt, rg, -(-C // 48))
