"""The forward's caller-owned workspace on the GPU.

- The size query is non-zero exactly for the kernels that use scratch memory
  (K split over workgroups; N:M rows expanded to dense codes), and a call with
  a workspace one byte short fails with ESIZE and launches nothing.
- Two streams run such calls at the same time, each with a workspace of its
  own: every result equals the oracle's bit for bit (acc) and within 1e-5
  (Y)."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import check_y, hip_pack, hip_quant, to_dev

pytestmark = pytest.mark.gpu

# (M, N, K, nm, kernel family using the workspace or None)
CASES = [
    (20, 4096, 6912, (0, 0), "splitk"),       # few tokens, K split over workgroups
    (40, 4096, 8192, (0, 0), "splitk"),
    (32, 2560, 6912, (2, 4), "splitk"),       # N:M t-byte GEMM with K split
    (512, 8960, 1536, (6, 8), "expand"),      # 6:8 prefill on expanded rows
    (100, 4100, 192, (2, 4), "expand"),       # 2:4 below 128 tokens
    (1, 6912, 2560, (0, 0), None),
    (8, 2048, 11008, (0, 0), None),
    (2048, 6912, 2560, (0, 0), None),
    (2048, 6912, 2560, (2, 4), None),         # sparse MFMA
]


@pytest.mark.parametrize("M,N,K,nm,family", CASES)
def test_size_query_names_the_scratch_kernels(M, N, K, nm, family):
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    print("case workspace query M=%d N=%d K=%d nm=%s" % (M, N, K, nm), flush=True)
    need = bl.forward_workspace_size(M, N, K, nm)
    W, X = workloads.small_case(3100 + M + K, M, N, K, outlier_frac=0.001)
    pk, ws = hip_pack(W, nm)
    Xq, xs, rs = hip_quant(X)
    Y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    if need:
        short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
        with pytest.raises(bl.BitLinearError) as ei:
            bl.forward(Xq, xs, rs, pk, ws, N, nm, Y=Y, workspace=short)
        assert ei.value.status == bl.binding.ESIZE
        torch.cuda.synchronize()
        assert bool((Y == 7.0).all()), "a rejected call wrote its output"
    Y, acc = bl.forward(Xq, xs, rs, pk, ws, N, nm, want_acc=True)
    name = bl.last_dispatch()
    if family is None:
        assert need == 0, (name, need)
    else:
        assert need > 0 and family in name, (name, need)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 40)).astype(int))
    beta, w_eff, _ = oracle.quantize_weights(W, *nm)
    q, xs_o, _ = oracle.quant_act(X[rows])
    acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
    assert np.array_equal(acc.cpu().numpy()[rows], acc_o)
    check_y(Y.cpu().numpy()[rows], Y_o, acc_o)


def test_two_streams_with_own_workspaces():
    # a split-K call and a 6:8 expand call, each repeated on its own stream
    # with its own workspace, issued interleaved without synchronisation
    import torch

    import oracle
    import ternary_weight_linear_act_amd as bl
    cases = [(20, 4096, 6912, (0, 0)), (512, 8960, 1536, (6, 8))]
    prep = []
    for i, (M, N, K, nm) in enumerate(cases):
        print("case two streams M=%d N=%d K=%d nm=%s" % (M, N, K, nm), flush=True)
        W, X = workloads.small_case(3300 + i, M, N, K, outlier_frac=0.001)
        pk, ws = hip_pack(W, nm)
        Xq, xs, rs = hip_quant(X)
        need = bl.forward_workspace_size(M, N, K, nm)
        assert need > 0
        prep.append(dict(W=W, X=X, M=M, N=N, K=K, nm=nm, pk=pk, ws=ws, Xq=Xq, xs=xs, rs=rs,
                         work=torch.empty(need, dtype=torch.uint8, device="cuda"),
                         Y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda"),
                         stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    for it in range(25):
        for c in prep:
            bl.forward(c["Xq"], c["xs"], c["rs"], c["pk"], c["ws"], c["N"], c["nm"], Y=c["Y"], acc=c["acc"],
                       workspace=c["work"], stream=c["stream"])
    torch.cuda.synchronize()
    for c in prep:
        rows = np.unique(np.linspace(0, c["M"] - 1, min(c["M"], 40)).astype(int))
        beta, w_eff, _ = oracle.quantize_weights(c["W"], *c["nm"])
        q, xs_o, _ = oracle.quant_act(c["X"][rows])
        acc_o, Y_o = oracle.forward(q, xs_o, w_eff, beta)
        assert np.array_equal(c["acc"].cpu().numpy()[rows], acc_o)
        check_y(c["Y"].cpu().numpy()[rows], Y_o, acc_o)
