"""bitlinear_forward_noalloc (the library's fixed per-GPU scratch instead of a
caller workspace) against bitlinear_forward on the same inputs, through the C
ABI: two calls in a row on each kernel family that uses scratch memory, the
second with a smaller input, each bit-identical (acc and Y) to the
workspace entry point's result; a call with no scratch; and a shape needing
more scratch than the array holds, rejected with ESIZE before anything runs."""
import numpy as np
import pytest

from ternary_weight_linear_act_amd import workloads

from gpu_helpers import hip_pack, hip_quant

pytestmark = pytest.mark.gpu


def run_pair(M, N, K, nm, seed):
    import torch

    import ternary_weight_linear_act_amd as bl
    print("case no-alloc M=%d N=%d K=%d nm=%s" % (M, N, K, nm), flush=True)
    W, X = workloads.small_case(seed, M, N, K, outlier_frac=0.001)
    pk, ws = hip_pack(W, nm)
    Xq, xs, rs = hip_quant(X)
    Y0, a0 = bl.forward(Xq, xs, rs, pk, ws, N, nm, want_acc=True)
    ref = bl.last_dispatch()
    Y1 = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    a1 = torch.full((M, N), 5, dtype=torch.int32, device="cuda")
    bl.forward_noalloc(Xq, xs, rs, pk, ws, N, nm, Y=Y1, acc=a1)
    assert bl.last_dispatch() == ref, (bl.last_dispatch(), ref)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1), "acc differs from bitlinear_forward's"
    assert torch.equal(Y0.view(torch.int32), Y1.view(torch.int32)), "Y differs from bitlinear_forward's"
    return ref, bl.forward_workspace_size(M, N, K, nm)


@pytest.mark.parametrize("first,second", [
    ((512, 8960, 1536, (6, 8)), (100, 2000, 1536, (6, 8))),     # N:M rows expanded in the scratch
    ((40, 4096, 8192, (0, 0)), (20, 4096, 6912, (0, 0))),       # K split, partial tiles in the scratch
    ((32, 2560, 6912, (2, 4)), (17, 8300, 512, (2, 4))),        # N:M t-byte GEMM with K split
    ((64, 2560, 6912, (0, 0)), (16, 2048, 11008, (0, 0))),      # token-tile kernel, K parts in the scratch
])
def test_noalloc_matches_forward_twice(first, second):
    # the second call is the smaller problem (its scratch use may differ: a
    # smaller prefill can split K); both use the array
    n1, w1 = run_pair(*first, seed=5100)
    n2, w2 = run_pair(*second, seed=5200)
    assert second[0] * second[2] < first[0] * first[2]          # M x K activations
    assert w1 > 0 and w2 > 0, (n1, w1, n2, w2)


def test_noalloc_without_scratch():
    name, w = run_pair(1, 2560, 6912, (0, 0), seed=5300)
    assert w == 0 and name.startswith("decode_dot4"), name


def test_noalloc_rejects_beyond_its_scratch():
    import torch

    import ternary_weight_linear_act_amd as bl
    M, N, K, nm = 100, 16384, 16384, (6, 8)
    assert bl.forward_workspace_size(M, N, K, nm) > 32 << 20
    pb, _ = bl.packed_size(N, K, nm)
    pk = torch.empty(pb, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(1, dtype=torch.float32, device="cuda")
    Xq = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    xs = torch.zeros(M, dtype=torch.float32, device="cuda")
    rs = torch.zeros(M, dtype=torch.int32, device="cuda")
    Y = torch.full((M, N), 2.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bl.BitLinearError) as ei:
        bl.forward_noalloc(Xq, xs, rs, pk, ws, N, nm, Y=Y)
    assert ei.value.status == bl.binding.ESIZE
    torch.cuda.synchronize()
    assert bool((Y == 2.0).all())
