"""GPU parity of the direct-load skinny forward with several 16-token tiles per
workgroup (dense weights at 9-64 tokens over at least 6912 weight rows, K of
4 to 48 chunks of 64): every dispatch rule at its token, row and K edges,
with ragged weight rows and a ragged last token group, against the CPU oracle
(acc bit-exact, Y within 1e-5); grouped calls bit-identical to the forward of
each projection alone; shapes just outside each rule take another kernel.
The form with K split over the workgroups (one projection, deep K): its K
range and row range at their edges, int32 partials in the caller's
workspace."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, cover_rows, direct_tiles, direct_tiles_split, full_check, hip_forward, hip_pack, hip_quant

pytestmark = pytest.mark.gpu


# (M, N, K) at the edges of each rule (one projection)
SINGLE = [
    (9, 6912, 256), (16, 7000, 2048), (12, 6913, 2112), (16, 6920, 3072),       # 9-16 tokens
    (17, 13824, 1024), (32, 14000, 3072), (25, 20000, 448),                     # 17-32, >= 13824 rows
    (17, 6912, 2048), (32, 13823, 2560), (20, 9000, 320),                       # 17-32, 6912-13823 rows
    (33, 16384, 256), (64, 16400, 2048), (48, 20000, 1088),                     # 33-64, >= 16384 rows
    (33, 6912, 3072), (64, 13823, 2560), (50, 8000, 512), (64, 11008, 2048),    # 33-64, 6912-13823 rows
    (17, 2560, 2560), (64, 6911, 3072), (40, 3000, 256), (64, 2560, 2560),      # 17-64, 2560-6911 rows
    (33, 2048, 2048), (64, 2559, 1024), (48, 2100, 3072),                       # 33-64, 2048-2559 rows
]


@pytest.mark.parametrize("M,N,K", SINGLE)
def test_tiles_single(M, N, K):
    import ternary_weight_linear_act_amd as bl
    want = direct_tiles(M, K, N)
    assert want is not None
    W, X = workloads.small_case(6100 + M + K + N, M, N, K, outlier_frac=0.001)
    full_check(W, X, (0, 0), rows=cover_rows(M), label="skinny-direct-tiles")
    assert bl.last_dispatch() == want, bl.last_dispatch()


@pytest.mark.parametrize("M,N,K,nm", [(8, 8200, 2048, (0, 0)), (9, 6911, 2048, (0, 0)), (16, 8200, 3136, (0, 0)),
                                      (17, 2559, 2048, (0, 0)), (16, 6000, 2048, (0, 0)), (32, 2048, 2048, (0, 0)),
                                      (64, 2047, 2048, (0, 0)),
                                      (33, 13824, 2048, (0, 0)), (33, 16384, 2112, (0, 0)), (65, 16384, 2048, (0, 0)),
                                      (24, 8200, 192, (0, 0)), (16, 8200, 2048, (2, 4)), (40, 8200, 2048, (6, 8))])
def test_tiles_outside_rules(M, N, K, nm):
    import ternary_weight_linear_act_amd as bl
    assert direct_tiles(M, K, N, nm) is None
    W, X = workloads.small_case(6200 + M + K + N, M, N, K, outlier_frac=0.001)
    full_check(W, X, nm, rows=cover_rows(M), label="skinny-direct-tiles-outside")
    assert not bl.last_dispatch().startswith("skinny_direct_tiles"), bl.last_dispatch()


@pytest.mark.parametrize("M,K,Ns", [(9, 1024, (3500, 3412)), (24, 2048, (3500, 3412)), (40, 512, (3500, 3412)),
                                    (16, 2560, (6912, 6912)), (32, 2560, (6912, 6912)), (33, 2048, (8200, 8200)),
                                    (64, 2048, (100, 16300)), (64, 1024, (2048,) * 8), (57, 3072, (7000, 33))])
def test_tiles_grouped(M, K, Ns):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    seed = 6300 + M + K + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 99, M, 8, K, outlier_frac=0.01)
    print("case direct tiles grouped M=%d K=%d Ns=%s" % (M, K, Ns), flush=True)
    want = direct_tiles(M, K, sum(Ns))
    assert want is not None
    packs = [hip_pack(W, (0, 0)) for W in Ws]
    Xq, xs, rs = hip_quant(X)
    projs = [(pk, ws, W.shape[0]) for (pk, ws), W in zip(packs, Ws)]
    Ys, accs = bl.forward_grouped(Xq, xs, rs, projs, want_acc=True)
    torch.cuda.synchronize()
    name = bl.last_dispatch()
    assert name == want + ("_grouped" if len(Ns) > 1 else ""), name
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


@pytest.mark.parametrize("M,N", [(40, 8200), (64, 16400)])
def test_tiles_extreme_accumulators_and_zero_rows(M, N):
    # q = -128 against t = -1 over the largest K of each K range, and an
    # all-zero token in the second token group
    import torch

    import ternary_weight_linear_act_amd as bl
    K = 3072 if N < 13824 else 2048
    W = np.full((N, K), -1.0, np.float32)
    packed, ws = hip_pack(W, (0, 0))
    Xq = torch.full((M, K), -128, dtype=torch.int8, device="cuda")
    Xq[19] = 0
    xs = torch.ones(M, dtype=torch.float32, device="cuda")
    rs = Xq.to(torch.int32).sum(1).to(torch.int32)
    Y, acc = hip_forward(Xq, xs, rs, packed, ws, N, (0, 0))
    torch.cuda.synchronize()
    assert bl.last_dispatch() == direct_tiles(M, K, N), bl.last_dispatch()
    a = acc.cpu().numpy()
    assert np.all(a[19] == 0) and np.all(np.delete(a, 19, axis=0) == 128 * K)
    assert not bool(Y[19].any())
    beta = ws.cpu().numpy()[0]
    assert np.all(Y.cpu().numpy()[np.arange(M) != 19] == np.float32(128 * K) * np.float32(beta))


# (M, N, K): 50, 108 and 384 chunks (2, 3 and 8 K parts), 1024 to 4096 rows
# (2560 past 32 tokens), ragged rows, 9 / 32 / 33 / 64 tokens, the 2B and 3B
# down projections (shapes the staged skinny kernel does not take)
SPLIT = [(9, 1024, 6912), (32, 1100, 24576), (32, 4096, 6912), (49, 2560, 3200), (33, 2049, 6912), (64, 2048, 11008),
         (16, 2560, 6912), (64, 2560, 6912), (20, 3000, 8192), (57, 1500, 7040)]


@pytest.mark.parametrize("M,N,K", SPLIT)
def test_tiles_split(M, N, K):
    import torch

    import ternary_weight_linear_act_amd as bl
    want = direct_tiles_split(M, K, N)
    assert want is not None and direct_tiles(M, K, N) is None
    W, X = workloads.small_case(6500 + M + K + N, M, N, K, outlier_frac=0.001)
    out = full_check(W, X, (0, 0), rows=cover_rows(M), label="skinny-direct-tiles-split")
    assert bl.last_dispatch() == want, bl.last_dispatch()
    # the partials live in the caller's workspace: the size query names it
    assert bl.forward_workspace_size(M, N, K, (0, 0)) >= int(want.rsplit("splitk", 1)[1]) * M * N * 4
    Y2, acc2 = hip_forward(out["Xq"], out["xs"], out["rs"], out["packed"], out["ws"], N, (0, 0))
    torch.cuda.synchronize()
    assert torch.equal(acc2, out["acc"]) and torch.equal(Y2.view(torch.int32), out["Y"].view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(8, 2048, 11008), (65, 2048, 11008), (16, 1023, 6912), (16, 4097, 6912),
                                   (64, 2048, 3072), (16, 2048, 24640), (33, 2561, 6912)])
def test_tiles_split_outside_rules(M, N, K):
    import ternary_weight_linear_act_amd as bl
    assert direct_tiles_split(M, K, N) is None
    W, X = workloads.small_case(6600 + M + K + N, M, N, K, outlier_frac=0.001)
    full_check(W, X, (0, 0), rows=cover_rows(M), label="skinny-direct-tiles-split-outside")
    name = bl.last_dispatch()
    assert "splitk" not in name or not name.startswith("skinny_direct_tiles"), name
    assert direct_tiles(M, K, N) is None or name == direct_tiles(M, K, N), name
