"""The hot path under HIP-graph capture, as bench.py times it.

Each case runs eagerly once, is captured into a graph on a side stream, and
is replayed three times with eager work (the outputs cleared) and a
synchronisation between the replays: every replay must equal the eager result
bit for bit.  The inputs are then overwritten in place: a replay must equal an
eager call on the new inputs, so the graph reads its buffers each time rather
than holding values from capture.  Covered: quant_act + forward (dense, 2:4,
6:8; one token, the few-token split-K kernel, the prefill tiles, the sparse
MFMA GEMM), the fused one-token launch with and without a row transform, the
fused 2-4-token launch, quant_act + the grouped forward (both skinny
kernels), quant_act_ex and the H-BitLinear quantiser.  And, in a
fresh process, forward calls captured before any eager call: the same kernels
and the same bits as the eager calls afterwards."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import hip_pack, to_dev

pytestmark = pytest.mark.gpu


def capture(body):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        body()
    torch.cuda.synchronize()
    return g


def check_replays(body, outs, refill):
    """body() eagerly, then its graph: 3 replays equal to the eager outputs;
    refill() overwrites the inputs, after which a replay equals body()."""
    import torch
    body()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = capture(body)
    for r in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), "replay %d differs from the eager result" % r
    refill()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = [o.clone() for o in outs]
    body()
    torch.cuda.synchronize()
    for o, e in zip(outs, got):
        assert torch.equal(o, e), "replay on new inputs differs from the eager call"
    assert not all(torch.equal(a, b) for a, b in zip(got, ref)), "new inputs gave the old outputs"


@pytest.mark.parametrize("M,N,K,nm", [(1, 2560, 6912, (0, 0)), (1, 6912, 2560, (2, 4)), (1, 2048, 2048, (6, 8)),
                                      (8, 2048, 11008, (0, 0)), (20, 4096, 6912, (0, 0)), (3, 300, 11008, (6, 8)),
                                      (40, 8200, 2048, (0, 0)),
                                      (64, 2048, 2048, (2, 4)), (512, 8960, 1536, (6, 8)),
                                      (2048, 6912, 2560, (0, 0)), (2048, 6912, 2560, (2, 4)),
                                      (1000, 8000, 640, (2, 4)), (300, 1000, 1472, (0, 0))])
def test_graph_two_call(M, N, K, nm):
    import torch

    import ternary_weight_linear_act_amd as bl
    W, X = workloads.small_case(2000 + M + K, M, N, K, outlier_frac=0.001)
    print("case graph two-call M=%d N=%d K=%d nm=%s" % (M, N, K, nm), flush=True)
    pk, ws = hip_pack(W, nm)
    Xd = to_dev(X)
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    rs = torch.empty(M, dtype=torch.int32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")

    def body():
        bl.quant_act(Xd, Xq, xs, rs)
        bl.forward(Xq, xs, rs, pk, ws, N, nm, Y=Y, acc=acc)

    X2 = workloads.activations(np.random.default_rng(2100 + M), M, K, 0.001)
    check_replays(body, [Xq, xs, rs, Y, acc], lambda: Xd.copy_(to_dev(X2)))


@pytest.mark.parametrize("M,tr", [(1, None), (1, "norm"), (1, "gate_norm"), (3, None)])
def test_graph_fused(M, tr):
    import torch

    import ternary_weight_linear_act_amd as bl
    K, Ns = 2560, (6912, 6912)
    rng = np.random.default_rng(2200 + M)
    Ws = [workloads.normal_f32(rng, (N, K), workloads.WEIGHT_SIGMA) for N in Ns]
    print("case graph fused M=%d tr=%s" % (M, tr), flush=True)
    packs = [hip_pack(W, (0, 0)) for W in Ws]
    Xd = to_dev(workloads.activations(rng, M, K, 0.001))
    up = to_dev(workloads.activations(rng, M, K)) if tr == "gate_norm" else None
    gamma = to_dev(rng.uniform(0.5, 1.5, K).astype(np.float32)) if tr else None
    Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for N in Ns]
    accs = [torch.empty((M, N), dtype=torch.int32, device="cuda") for N in Ns]
    xs = torch.empty(M, dtype=torch.float32, device="cuda")

    def body():
        bl.forward_fused_ex(Xd, [(pk, ws, N) for (pk, ws), N in zip(packs, Ns)], up=up, gamma=gamma,
                            eps=1e-5 if tr else None, Ys=Ys, accs=accs, x_scale=xs)

    X2 = workloads.activations(rng, M, K, 0.001)
    check_replays(body, Ys + accs + [xs], lambda: Xd.copy_(to_dev(X2)))


@pytest.mark.parametrize("M,Ns,K", [(8, (11008, 11008), 2048), (64, (2048, 256, 256), 2048), (16, (300, 17), 512),
                                    (64, (11008, 11008), 2048)])
def test_graph_grouped(M, Ns, K):
    # quant_act + the grouped forward (one launch per input group), as the
    # bench runs the 3B block past 4 tokens: the direct-load kernel at 8 and
    # 64 tokens, the staged one at 16, the few-token GEMM for gate + up at 64
    import torch

    import ternary_weight_linear_act_amd as bl
    rng = np.random.default_rng(2250 + M)
    Ws = [workloads.normal_f32(rng, (N, K), workloads.WEIGHT_SIGMA) for N in Ns]
    print("case graph grouped M=%d Ns=%s K=%d" % (M, Ns, K), flush=True)
    packs = [hip_pack(W, (0, 0)) for W in Ws]
    Xd = to_dev(workloads.activations(rng, M, K, 0.001))
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    rs = torch.empty(M, dtype=torch.int32, device="cuda")
    Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for N in Ns]
    accs = [torch.empty((M, N), dtype=torch.int32, device="cuda") for N in Ns]

    def body():
        bl.quant_act(Xd, Xq, xs, rs)
        bl.forward_grouped(Xq, xs, rs, [(pk, ws, N) for (pk, ws), N in zip(packs, Ns)], Ys=Ys, accs=accs)

    X2 = workloads.activations(rng, M, K, 0.001)
    check_replays(body, Ys + accs + [Xq, xs, rs], lambda: Xd.copy_(to_dev(X2)))


@pytest.mark.parametrize("kind", ["quant_act_ex", "quant_act_h4"])
def test_graph_quantisers(kind):
    import torch

    import ternary_weight_linear_act_amd as bl
    M, K = 37, 6912
    rng = np.random.default_rng(2300)
    print("case graph %s" % kind, flush=True)
    Xd = to_dev(workloads.activations(rng, M, K, 0.01))
    up = to_dev(workloads.activations(rng, M, K))
    gamma = to_dev(rng.uniform(0.25, 1.75, K).astype(np.float32))
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    rs = torch.empty(M, dtype=torch.int32, device="cuda")

    def body():
        if kind == "quant_act_ex":
            bl.quant_act_ex(Xd, up, gamma, 1e-5, Xq=Xq, x_scale=xs, x_rowsum=rs)
        else:
            bl.quant_act_h4(Xd, 256, Xq, xs, rs)

    X2 = workloads.activations(rng, M, K, 0.01)
    check_replays(body, [Xq, xs, rs], lambda: Xd.copy_(to_dev(X2)))


_FIRST_CALL_CAPTURED = r'''
import numpy as np
import torch
import ternary_weight_linear_act_amd as bl
from ternary_weight_linear_act_amd import workloads
# a 6:8 prefill (rows expanded in the workspace) and a few-token GEMM with K
# split over workgroups (partial sums in the workspace)
cases = [(512, 8960, 1536, (6, 8)), (20, 4096, 6912, (0, 0))]
dev = torch.device("cuda:0")
prep = []
for M, N, K, nm in cases:
    W, X = workloads.small_case(2400 + M, M, N, K, outlier_frac=0.001)
    pk, ws = bl.pack_weights(torch.from_numpy(W).to(dev), nm)
    Xq, xs, rs = bl.quant_act(torch.from_numpy(X).to(dev))
    prep.append((M, N, K, nm, pk, ws, Xq, xs, rs, torch.empty((M, N), dtype=torch.float32, device=dev),
                 torch.empty((M, N), dtype=torch.int32, device=dev)))
    assert bl.forward_workspace_size(M, N, K, nm) > 0
torch.cuda.synchronize()
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
g = torch.cuda.CUDAGraph()
names = []
with torch.cuda.graph(g, stream=s):                  # the first forward calls of the process
    for M, N, K, nm, pk, ws, Xq, xs, rs, Y, acc in prep:
        bl.forward(Xq, xs, rs, pk, ws, N, nm, Y=Y, acc=acc)
        names.append(bl.last_dispatch())
g.replay()
torch.cuda.synchronize()
for i, (M, N, K, nm, pk, ws, Xq, xs, rs, Y, acc) in enumerate(prep):
    Yg, ag = Y.clone(), acc.clone()
    Ye, ae = bl.forward(Xq, xs, rs, pk, ws, N, nm, want_acc=True)
    eager = bl.last_dispatch()
    torch.cuda.synchronize()
    print("case", M, N, K, nm, "captured:", names[i], "eager:", eager, flush=True)
    assert names[i] == eager, "the captured call took another kernel"
    assert "splitk" in eager or "expand" in eager, eager
    assert torch.equal(ag, ae) and torch.equal(Yg, Ye)
print("ok", flush=True)
'''


def test_graph_first_call_same_kernel():
    # in a fresh process, forward calls captured before any eager call take
    # the same kernels as the eager calls made afterwards (the kernel choice
    # depends on the shape alone; the workspace comes from the caller, here
    # torch's graph pool) and give the same bits
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED], cwd=root, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
