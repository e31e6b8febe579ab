"""Benchmark of the BitLinear forward on one MI355X.

Headline: BitLinear GB/s at M = 1 (decode GEMV over a 2B-class FFN: gate and up
2560 -> 6912, down 6912 -> 2560) as a fraction of HBM peak, and int8 TOPS at
M = 2048 (prefill GEMM, K = 2560, N = 6912) as a fraction of int8 MFMA peak.

A step is one pass of the hot path over one batch: for each projection,
per-token int8 activation quantisation, then the packed-ternary forward with
its fused dequant epilogue.  Weights are packed once, outside the timed
region (they are stored packed).  The packed weights rotate through a pool of
distinct buffers larger than the 256 MB Infinity Cache so that every step
streams its weights from HBM.  Steps are captured in a HIP graph and timed
with HIP events on the capture's stream, bracketed by device synchronisation.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
                       [--traffic-probe] [--gemm-probe]
Prints one JSON line on stdout; a readable summary goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POP/s)
POOL_BYTES = 512 << 20         # >= 2x the 256 MB Infinity Cache

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_decode_ffn_2b.json")
CSRC = os.path.join(ROOT, "ternary_weight_linear_act_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def fwd_bytes(M, N, K, nm=(0, 0)):
    """Algorithmic bytes of one forward launch: packed weights, int8 activations,
    x_scale + row sums, beta, fp32 output."""
    wbytes = N * K * (5 / 16 if nm == (6, 8) else 1 / 4)
    return int(wbytes + M * K + 8 * M + 4 + 4 * M * N)


def quant_bytes(M, K):
    """fp32 in, int8 out, x_scale and row sum."""
    return 4 * M * K + M * K + 8 * M


def timed_graph(torch, body, reps=1, warm=1):
    """Capture body() into a HIP graph, replay it `warm` times untimed, then
    time `reps` replays with events on the graph's stream.  Returns ms per
    replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()                                   # eager warm call outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        body()
    # replay on s and record the events on s: graph launches go to the current stream
    with torch.cuda.stream(s):
        for _ in range(warm):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps, g


def bench_configs(torch, bl, workloads, dev, log):
    """The other workloads, reported beside the headline (not part of `value`):
    single_1024 (M = 1, 16), sparse_ffn_1p5b (dense / 2:4 / 6:8 at M = 1 and
    512) and block_3b (seven projections at M = 1, 8, 64).  HBM-bound cases
    rotate weight copies through >= 512 MB; each case is checked against the
    plain path before it is timed (fused == two-call, bit for bit)."""
    res = {}

    def case(name, wl_name, projs, M, nm_of, fused_groups=None):
        wl = workloads.WORKLOADS[wl_name]
        d = workloads.draw(wl_name, projs=projs, Ms=(M,))
        shapes = {p.name: (p.N, p.K) for p in wl.projs if p.name in projs}
        pk, ws = {}, {}
        for n in projs:
            pk[n], ws[n] = bl.pack_weights(torch.from_numpy(d.W[n]).to(dev), nm=nm_of(n))
        wbytes = sum(pk[n].numel() for n in projs)
        P = max(2, -(-POOL_BYTES // wbytes)) if M <= 64 else 1
        pools = {n: [pk[n]] + [pk[n].clone() for _ in range(P - 1)] for n in projs}
        X = {n: torch.from_numpy(d.X[(n, M)]).to(dev) for n in projs}
        Y = {n: torch.empty((M, shapes[n][0]), dtype=torch.float32, device=dev) for n in projs}
        Xq = {n: torch.empty((M, shapes[n][1]), dtype=torch.int8, device=dev) for n in projs}
        xs = {n: torch.empty(M, dtype=torch.float32, device=dev) for n in projs}
        rs = {n: torch.empty(M, dtype=torch.int32, device=dev) for n in projs}

        def two_call(j):
            for n in projs:
                bl.quant_act(X[n], Xq[n], xs[n], rs[n])
                bl.forward(Xq[n], xs[n], rs[n], pools[n][j], ws[n], shapes[n][0], nm=nm_of(n), Y=Y[n])
        two_call(0)
        torch.cuda.synchronize()
        Yref = {n: Y[n].clone() for n in projs}
        kernels = sorted({bl.last_dispatch()})
        G = P if M <= 64 else 10
        ms, _ = timed_graph(torch, lambda: [two_call(j % P) for j in range(G)], reps=2)
        us = ms * 1e3 / G
        abytes = sum(pk[n].numel() + shapes[n][1] * M * 4 + M * shapes[n][0] * 4 for n in projs)
        ops = sum(2.0 * M * shapes[n][0] * shapes[n][1] for n in projs)
        r = {"M": M, "projections": list(projs), "two_call_us": round(us, 3),
             "two_call_GB/s": round(abytes / (us * 1e-6) / 1e9, 1), "TOPS": round(ops / (us * 1e-6) / 1e12, 1)}
        if fused_groups and M <= 4:
            def fused(j):
                for g in fused_groups:
                    bl.forward_fused(X[g[0]], [(pools[n][j], ws[n], shapes[n][0]) for n in g], nm=nm_of(g[0]),
                                     Ys=[Y[n] for n in g])
            fused(0)
            torch.cuda.synchronize()
            for n in projs:
                if not torch.equal(Y[n], Yref[n]):
                    raise SystemExit("%s: fused and two-call outputs differ for %s" % (name, n))
            ms, _ = timed_graph(torch, lambda: [fused(j % P) for j in range(G)], reps=2)
            fus = ms * 1e3 / G
            fbytes = sum(pk[n].numel() + M * shapes[n][0] * 4 for n in projs) + sum(
                4 * M * shapes[g[0]][1] for g in fused_groups)
            r.update({"fused_us": round(fus, 3), "fused_GB/s": round(fbytes / (fus * 1e-6) / 1e9, 1),
                      "fused_launches": len(fused_groups)})
        res[name] = r
        log("%-28s M=%-4d two-call %8.2f us%s" % (name, M, us, (" fused %.2f us" % r["fused_us"]) if "fused_us" in r else ""))

    dense = lambda n: (0, 0)
    case("single_1024/M1", "single_1024", ("linear",), 1, dense, [("linear",)])
    case("single_1024/M16", "single_1024", ("linear",), 16, dense)
    nmap = {"dense": (0, 0), "nm24": (2, 4), "nm68": (6, 8)}
    for pn in ("dense", "nm24", "nm68"):
        case("sparse_ffn_1p5b/%s/M1" % pn, "sparse_ffn_1p5b", (pn,), 1, lambda n: nmap[n], [(pn,)])
        case("sparse_ffn_1p5b/%s/M512" % pn, "sparse_ffn_1p5b", (pn,), 512, lambda n: nmap[n])
    blk = ("q", "k", "v", "o", "gate", "up", "down")
    for M in (1, 8, 64):
        case("block_3b/M%d" % M, "block_3b", blk, M, dense,
             [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)])
    return res


def bench_ffn_block(torch, bl, dev, log, x_pool, shapes, packed, wsc, P):
    """The feed-forward block of the decode step with the steps either side of
    the linears fused in: RMSNorm -> gate, up (one launch), then ReLU^2(gate) *
    up -> subln RMSNorm -> down (one launch), against the same on the two-call
    path (quant_act_ex, then forward per projection: five launches).  Same
    weight pool as the decode step; RMSNorm weights uniform in [0.5, 1.5]."""
    import numpy as np
    (F, D), eps = shapes["gate"], 1e-5
    rng = np.random.default_rng(7)
    g_in = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).to(dev)
    g_sub = torch.from_numpy(rng.uniform(0.5, 1.5, F).astype(np.float32)).to(dev)
    G = torch.empty((1, F), dtype=torch.float32, device=dev)
    U = torch.empty_like(G)
    Yd = torch.empty((1, D), dtype=torch.float32, device=dev)
    names = []

    def fused(j):
        bl.forward_fused_ex(x_pool[j], [(packed["gate"][j], wsc["gate"], F), (packed["up"][j], wsc["up"], F)],
                            gamma=g_in, eps=eps, Ys=[G, U])
        names.append(bl.last_dispatch())
        bl.forward_fused_ex(G, [(packed["down"][j], wsc["down"], D)], up=U, gamma=g_sub, eps=eps, Ys=[Yd])
        names.append(bl.last_dispatch())

    Xq1, Xq2 = torch.empty((1, D), dtype=torch.int8, device=dev), torch.empty((1, F), dtype=torch.int8, device=dev)
    xs = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(2)]
    rs = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(2)]
    G2, U2, Y2 = torch.empty_like(G), torch.empty_like(U), torch.empty_like(Yd)

    def two_call(j):
        bl.quant_act_ex(x_pool[j], gamma=g_in, eps=eps, Xq=Xq1, x_scale=xs[0], x_rowsum=rs[0])
        bl.forward(Xq1, xs[0], rs[0], packed["gate"][j], wsc["gate"], F, Y=G2)
        bl.forward(Xq1, xs[0], rs[0], packed["up"][j], wsc["up"], F, Y=U2)
        bl.quant_act_ex(G2, up=U2, gamma=g_sub, eps=eps, Xq=Xq2, x_scale=xs[1], x_rowsum=rs[1])
        bl.forward(Xq2, xs[1], rs[1], packed["down"][j], wsc["down"], D, Y=Y2)

    fused(0)
    two_call(0)
    torch.cuda.synchronize()
    kernels = names[:2]
    # the two paths agree up to the one-ulp latitude of the norm's scale (the
    # down stage compared on the same inputs: the fused path's gate and up)
    bl.quant_act_ex(G, up=U, gamma=g_sub, eps=eps, Xq=Xq2, x_scale=xs[1], x_rowsum=rs[1])
    bl.forward(Xq2, xs[1], rs[1], packed["down"][0], wsc["down"], D, Y=Y2)
    for a, b in ((G, G2), (U, U2), (Yd, Y2)):
        if not torch.allclose(a, b, rtol=2e-6, atol=0.0):
            raise SystemExit("ffn block: fused and two-call outputs differ")
    ms_f, _ = timed_graph(torch, lambda: [fused(j % P) for j in range(P)], reps=3)
    ms_t, _ = timed_graph(torch, lambda: [two_call(j % P) for j in range(P)], reps=2)
    fus, two = ms_f * 1e3 / P, ms_t * 1e3 / P
    wbytes = sum(shapes[n][0] * shapes[n][1] // 4 for n in ("gate", "up", "down"))
    # weights; x and gamma_in read; gate and up written, then read with gamma_sub; y written
    abytes = wbytes + 4 * D * 2 + 4 * F * 2 + 4 * F * 3 + 4 * D
    log("ffn block (norm + gate/up, ReLU^2 + norm + down) fused %.2f us, two-call %.2f us" % (fus, two))
    return {"workload": "decode_ffn_2b with RMSNorm before gate/up, ReLU^2(gate)*up and subln RMSNorm before "
                        "down, M=1, weights rotating over %d buffers" % P,
            "fused_us": round(fus, 3), "fused_GB/s": round(abytes / (fus * 1e-6) / 1e9, 1), "fused_launches": 2,
            "kernels": kernels, "two_call_us": round(two, 3), "two_call_launches": 5}


def bench_h4(torch, bl, dev, log):
    """The H-BitLinear path on the down projection of the 2B-class FFN
    (6912 -> 2560, Hadamard blocks of 256): bitlinear_quant_act_h4, then
    bitlinear_forward, at one token (weights rotating through >= 512 MB) and
    at 2048 tokens, beside the 8-bit two-call path on the same shapes."""
    import numpy as np
    N, K, B = 2560, 6912, 256
    rng = np.random.default_rng(11)
    from ternary_weight_linear_act_amd import workloads
    W = workloads.normal_f32(rng, (N, K), workloads.WEIGHT_SIGMA)
    pk, ws = bl.pack_weights(torch.from_numpy(W).to(dev))
    res = {}
    for M in (1, 2048):
        X = torch.from_numpy(workloads.activations(rng, M, K, 0.001)).to(dev)
        P = max(2, -(-POOL_BYTES // pk.numel())) if M == 1 else 1
        pool = [pk] + [pk.clone() for _ in range(P - 1)]
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        xs = torch.empty(M, dtype=torch.float32, device=dev)
        rs = torch.empty(M, dtype=torch.int32, device=dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        G = P if M == 1 else 10
        t = {}
        for name, quant in (("h4", lambda: bl.quant_act_h4(X, B, Xq, xs, rs)),
                            ("int8", lambda: bl.quant_act(X, Xq, xs, rs))):
            quant()
            qkern = bl.last_dispatch()
            fw = lambda j: bl.forward(Xq, xs, rs, pool[j % P], ws, N, Y=Y)
            fw(0)
            torch.cuda.synchronize()
            ms_q, _ = timed_graph(torch, lambda: [quant() for _ in range(G)], reps=2)
            ms_f, _ = timed_graph(torch, lambda: [fw(j) for j in range(G)], reps=2)
            ms_s, _ = timed_graph(torch, lambda: [(quant(), fw(j)) for j in range(G)], reps=2)
            t[name] = {"quant_kernel": qkern, "quant_us": round(ms_q * 1e3 / G, 3),
                       "forward_us": round(ms_f * 1e3 / G, 3),
                       "step_us": round(ms_s * 1e3 / G, 3)}
        res["down_6912x2560_M%d" % M] = t
        log("h-bitlinear down M=%d: h4 step %.2f us (quant %.2f), int8 step %.2f us" % (
            M, t["h4"]["step_us"], t["h4"]["quant_us"], t["int8"]["step_us"]))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' timings")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a few eager decode steps and a copy kernel of known size, then exit "
                         "(the command profiled with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="run the prefill GEMM (2048 x 2560 -> 6912, dense) five times eagerly, then exit "
                         "(the command profiled with rocprofv3 --pmc for its SQ counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_linear_act_amd as bl
    from ternary_weight_linear_act_amd import workloads

    bl.load_library()                      # raises if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log("device: %s (%s), %d CUs" % (props.name, getattr(props, "gcnArchName", "?"), props.multi_processor_count))

    if args.gemm_probe:
        dp = workloads.draw("prefill_2048")
        pk_p, ws_p = bl.pack_weights(torch.from_numpy(dp.W["up"]).to(dev))
        Xq_p, xs_p, rs_p = bl.quant_act(torch.from_numpy(dp.X[("up", 2048)]).to(dev))
        Y_p = torch.empty((2048, 6912), dtype=torch.float32, device=dev)
        for _ in range(5):
            bl.forward(Xq_p, xs_p, rs_p, pk_p, ws_p, 6912, Y=Y_p)
        torch.cuda.synchronize()
        log("gemm probe: 5 launches of %s" % bl.last_dispatch())
        print(json.dumps({"gemm_launches": 5, "kernel": bl.last_dispatch(), "source_digest": source_digest()}),
              flush=True)
        return

    # ------------------------------------------------------------------ decode
    # One decode step of a 2B-class FFN at M = 1: the fused call (activation
    # quantisation + projections sharing the input, one launch) for gate/up,
    # then for down.  Weights rotate through a pool > 2x the Infinity Cache.
    wl = workloads.WORKLOADS["decode_ffn_2b"]
    d = workloads.draw("decode_ffn_2b")
    shapes = {p.name: (p.N, p.K) for p in wl.projs}
    groups = workloads.input_groups(wl)
    step_w_bytes = sum(N * K // 4 for N, K in shapes.values())
    P = max(2, -(-POOL_BYTES // step_w_bytes))
    packed, wsc, Y = {}, {}, {}
    for name, (N, K) in shapes.items():
        pk, ws = bl.pack_weights(torch.from_numpy(d.W[name]).to(dev))
        packed[name] = [pk] + [pk.clone() for _ in range(P - 1)]
        wsc[name] = ws
        Y[name] = torch.empty((1, N), dtype=torch.float32, device=dev)
    Xg = {}
    for g in groups:
        X = torch.from_numpy(d.X[(g[0], 1)]).to(dev)
        Xg[g] = [X] + [X.clone() for _ in range(P - 1)]
    torch.cuda.synchronize()
    log("decode: pool of %d weight sets, %.0f MB" % (P, P * step_w_bytes / 1e6))

    def decode_step(i):
        j = i % P
        for g in groups:
            bl.forward_fused(Xg[g][j], [(packed[n][j], wsc[n], shapes[n][0]) for n in g],
                             Ys=[Y[n] for n in g])

    # gate before timing: the kernel choice; the values are checked against
    # the oracle in the CPU leg below (and by the GPU tests)
    group_kernel = {}
    for g in groups:
        bl.forward_fused(Xg[g][0], [(packed[n][0], wsc[n], shapes[n][0]) for n in g], Ys=[Y[n] for n in g])
        group_kernel["+".join(g)] = bl.last_dispatch()
    torch.cuda.synchronize()
    for g, k in group_kernel.items():
        if not k.startswith("fused_decode"):
            raise SystemExit("unexpected kernel for the M=1 decode step (%s): %s" % (g, k))
    dispatch = ", ".join("%s: %s" % gk for gk in group_kernel.items())
    decode_Y = {name: Y[name].cpu().numpy().astype(np.float64) for name in shapes}

    if args.traffic_probe:
        # counters per dispatch: 2 x P eager decode steps over the rotating pool,
        # then a byte copy of COPY_BYTES (reads and writes that many bytes) as
        # the calibration of FETCH_SIZE / WRITE_SIZE
        for i in range(2 * P):
            decode_step(i)
        copy_bytes = 256 << 20
        src = torch.full((copy_bytes,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("traffic probe: %d fused decode launches, then a %d-byte device copy" % (2 * P * len(groups), copy_bytes))
        print(json.dumps({"fused_launches": 2 * P * len(groups), "copy_bytes": copy_bytes,
                          "source_digest": source_digest()}), flush=True)
        return

    def group_bytes(g):
        N0, K = shapes[g[0]]
        return 4 * K + 4 + sum(shapes[n][0] * K // 4 + 4 + 4 * shapes[n][0] for n in g)
    step_bytes = sum(group_bytes(g) for g in groups)

    # warmup W steps, then exactly K steps, each captured as one graph
    if args.warmup > 0:
        timed_graph(torch, lambda: [decode_step(i) for i in range(args.warmup)])
    torch.cuda.synchronize()
    ms_total, _ = timed_graph(torch, lambda: [decode_step(i) for i in range(args.steps)])
    ms_step = ms_total / args.steps
    value_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: the fused decode kernel; R launches over the rotating pool
    R = len(groups) * P
    ms_fused, _ = timed_graph(torch, lambda: [decode_step(i) for i in range(P)], reps=3)
    fused_us = ms_fused * 1e3 / R
    fused_gbs = step_bytes * P / (ms_fused * 1e-3) / 1e9
    per_group = {}
    for g in groups:
        def one(g=g):
            for j in range(P):
                bl.forward_fused(Xg[g][j], [(packed[n][j], wsc[n], shapes[n][0]) for n in g],
                                 Ys=[Y[n] for n in g])
        ms, _ = timed_graph(torch, one, reps=3)
        per_group["+".join(g)] = {"kernel": group_kernel["+".join(g)], "us": round(ms * 1e3 / P, 3),
                                  "GB/s": round(group_bytes(g) / (ms * 1e-3 / P) / 1e9, 1)}

    # context: the two-call path (quant_act, then forward per projection)
    Xq1, xs1, rs1 = {}, {}, {}
    for g in groups:
        K = shapes[g[0]][1]
        Xq1[g] = torch.empty((1, K), dtype=torch.int8, device=dev)
        xs1[g] = torch.empty(1, dtype=torch.float32, device=dev)
        rs1[g] = torch.empty(1, dtype=torch.int32, device=dev)

    def two_call_step(i):
        j = i % P
        for g in groups:
            bl.quant_act(Xg[g][j], Xq1[g], xs1[g], rs1[g])
            for n in g:
                bl.forward(Xq1[g], xs1[g], rs1[g], packed[n][j], wsc[n], shapes[n][0], Y=Y[n])
    ms_two, _ = timed_graph(torch, lambda: [two_call_step(i) for i in range(P)], reps=2)
    two_call_us = ms_two * 1e3 / P
    single = {}
    for name in ("up", "down"):
        N, K = shapes[name]
        g = [gg for gg in groups if name in gg][0]
        def fw(name=name, N=N, g=g):
            for j in range(P):
                bl.forward(Xq1[g], xs1[g], rs1[g], packed[name][j], wsc[name], N, Y=Y[name])
        ms, _ = timed_graph(torch, fw, reps=3)
        fb = N * K // 4 + K + 12 + 4 * N
        single["%dx%d" % (K, N)] = {"kernel": bl.last_dispatch(), "us": round(ms * 1e3 / P, 3),
                                    "GB/s": round(fb / (ms * 1e-3 / P) / 1e9, 1)}

    ffn_block = bench_ffn_block(torch, bl, dev, log, Xg[groups[0]], shapes, packed, wsc, P)
    h4 = bench_h4(torch, bl, dev, log)

    # ------------------------------------------------------------------ prefill
    dp = workloads.draw("prefill_2048")
    Wp = torch.from_numpy(dp.W["up"]).to(dev)
    Xp = torch.from_numpy(dp.X[("up", 2048)]).to(dev)
    Mp, Np_, Kp = 2048, 6912, 2560
    pk_p, ws_p = bl.pack_weights(Wp)
    Xq_p, xs_p, rs_p = bl.quant_act(Xp)
    Y_p = torch.empty((Mp, Np_), dtype=torch.float32, device=dev)
    bl.forward(Xq_p, xs_p, rs_p, pk_p, ws_p, Np_, Y=Y_p)
    torch.cuda.synchronize()
    gemm_dispatch = bl.last_dispatch()
    G = 20
    # steady state: ~5 ms of the same GEMM untimed first (the first
    # milliseconds of back-to-back GEMMs run a few percent slower), then 100
    # timed launches
    ms_gemm, _ = timed_graph(torch, lambda: [bl.forward(Xq_p, xs_p, rs_p, pk_p, ws_p, Np_, Y=Y_p) for _ in range(G)],
                             reps=5, warm=5)
    gemm_us = ms_gemm * 1e3 / G
    gemm_tops = 2.0 * Mp * Np_ * Kp / (gemm_us * 1e-6) / 1e12
    ms_qp, _ = timed_graph(torch, lambda: [bl.quant_act(Xp, Xq_p, xs_p, rs_p) for _ in range(G)], reps=2)
    quant_p_us = ms_qp * 1e3 / G
    # the same prefill with 2:4 weights (sparse MFMA); sampled accumulator rows
    # of both are kept for the oracle check in the CPU leg
    rows = np.array([0, 1, 777, 1500, Mp - 1])
    acc_p = torch.empty((Mp, Np_), dtype=torch.int32, device=dev)
    bl.forward(Xq_p, xs_p, rs_p, pk_p, ws_p, Np_, Y=Y_p, acc=acc_p)
    pk_s, ws_s = bl.pack_weights(Wp, nm=(2, 4))
    Y_s = torch.empty_like(Y_p)
    acc_s = torch.empty((Mp, Np_), dtype=torch.int32, device=dev)
    bl.forward(Xq_p, xs_p, rs_p, pk_s, ws_s, Np_, nm=(2, 4), Y=Y_s, acc=acc_s)
    torch.cuda.synchronize()
    gemm24_dispatch = bl.last_dispatch()
    prefill_rows = {"dense": acc_p.cpu().numpy()[rows], "2:4": acc_s.cpu().numpy()[rows]}
    ms_g24, _ = timed_graph(torch, lambda: [bl.forward(Xq_p, xs_p, rs_p, pk_s, ws_s, Np_, nm=(2, 4), Y=Y_s)
                                            for _ in range(G)], reps=5, warm=5)
    gemm24_us = ms_g24 * 1e3 / G
    # context: the vendor int8 GEMM (hipBLASLt through torch._int_mm) on the
    # same codes with the weights unpacked to one int8 per weight, K-major
    # (its faster layout here); int32 out, no dequant epilogue
    lib = None
    try:
        # the weights as int8, read back through the library itself: codes of
        # an identity activation block (row k = e_k, row sum 1, scale 1) give
        # acc[k, n] = W_eff[n, k]
        eye = torch.eye(Kp, dtype=torch.int8, device=dev)
        wt = torch.empty((Kp, Np_), dtype=torch.int32, device=dev)
        bl.forward(eye, torch.ones(Kp, dtype=torch.float32, device=dev),
                   torch.ones(Kp, dtype=torch.int32, device=dev), pk_p, ws_p, Np_, acc=wt)
        Bm = wt.t().contiguous().to(torch.int8).t()           # K x N view of an N x K matrix
        del wt, eye
        C = torch._int_mm(Xq_p, Bm)
        torch.cuda.synchronize()
        if not torch.equal(C, acc_p):
            raise RuntimeError("library int8 GEMM result differs from the accumulators")
        ms_lib, _ = timed_graph(torch, lambda: [torch._int_mm(Xq_p, Bm) for _ in range(G)], reps=5, warm=5)
        lib = {"op": "torch._int_mm (hipBLASLt), int8 x int8 -> int32, weights unpacked to int8, no epilogue",
               "us": round(ms_lib * 1e3 / G, 2),
               "TOPS": round(2.0 * Mp * Np_ * Kp / (ms_lib * 1e-3 / G) / 1e12, 1)}
        del Bm, C
    except (RuntimeError, AttributeError) as e:
        lib = {"op": "torch._int_mm", "error": str(e)[:200]}

    # ------------------------------------------------------------------ traffic
    traffic = None
    digest = source_digest()
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE))
            if t.get("source_digest") == digest:
                traffic = t.get("hbm_bytes_per_launch")
        except (ValueError, OSError):
            traffic = None

    # ------------------------------------------------------------------ other workloads
    configs = None if args.no_configs else bench_configs(torch, bl, workloads, dev, log)

    # ------------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle, timed on a bounded sample of the decode workload; its
        # outputs on that sample (and on sampled prefill rows) are compared
        # with what the GPU produced above
        import oracle
        pre = {}
        for name in shapes:
            beta, w_eff, _ = oracle.quantize_weights(d.W[name])
            pre[name] = (beta, w_eff)
        n = 0
        t0 = time.perf_counter()
        while True:
            for g in groups:
                q, xso, _ = oracle.quant_act(d.X[(g[0], 1)])
                for name in g:
                    oracle.forward(q, xso, pre[name][1], pre[name][0])
            n += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        cpu_s = (time.perf_counter() - t0) / n
        for name in shapes:
            q, xso, _ = oracle.quant_act(d.X[(name, 1)])
            _, Yo = oracle.forward(q, xso, pre[name][1], pre[name][0])
            if not np.all(np.abs(decode_Y[name] - Yo) <= 1e-5 * np.abs(Yo)):
                raise SystemExit("decode output of %s does not match the oracle" % name)
        q_p, xs_po, _ = oracle.quant_act(dp.X[("up", 2048)][rows])
        for kind, (n_, m_) in (("dense", (0, 0)), ("2:4", (2, 4))):
            beta_p, w_eff_p, _ = oracle.quantize_weights(dp.W["up"], n_, m_)
            acc_o, _ = oracle.forward(q_p, xs_po, w_eff_p, beta_p)
            if not np.array_equal(prefill_rows[kind], acc_o):
                raise SystemExit("%s prefill accumulators do not match the oracle" % kind)
        cpu = {"value": round(step_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "%d oracle decode steps (quantisation of the gate/up and down inputs, forward of "
                         "gate, up, down at M=1, the same seeded inputs), %.1f s, single-threaded C on %s" % (
                             n, n * cpu_s, platform.processor() or "host CPU"),
               "ms_per_step": round(cpu_s * 1e3, 3)}

    out = {
        "metric": "BitLinear GB/s @M=1 and int8 TOPS @M=2048, as % of MI355X roofline",
        "value": round(value_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xternary->int32->fp32",
        "data": "synthetic (seeded N(0,0.02) latent weights, N(0,1) activations with 0.1% x20 outliers)",
        "config": {"workload": "decode_ffn_2b: M=1, gate/up 2560->6912 (shared input), down 6912->2560; "
                               "per step one fused launch (int8 quantisation + projections) per input group; "
                               "weights rotating over %d buffers (%.0f MB)" % (P, P * step_w_bytes / 1e6),
                   "M": 1, "projections": ["gate 2560x6912", "up 2560x6912", "down 6912x2560"]},
        "roofline": {"bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fused_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": dispatch, "avg_launch_us": round(fused_us, 3),
                     "bytes_per_launch": round(step_bytes / len(groups)), "per_group": per_group},
        "decode_two_call_path": {"step_us": round(two_call_us, 3),
                                 "GB/s": round(step_bytes / (two_call_us * 1e-6) / 1e9, 1),
                                 "single_forward": single},
        "gemm": {"workload": "prefill_2048: M=2048, K=2560, N=6912", "kernel": gemm_dispatch,
                 "avg_launch_us": round(gemm_us, 2), "TOPS": round(gemm_tops, 1),
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS,
                              "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4)},
                 "quant_act_us": round(quant_p_us, 2),
                 "nm24": {"kernel": gemm24_dispatch, "avg_launch_us": round(gemm24_us, 2),
                          "TOPS_dense_equivalent": round(2.0 * Mp * Np_ * Kp / (gemm24_us * 1e-6) / 1e12, 1),
                          "vs_dense": round(gemm_us / gemm24_us, 3)},
                 "library_int8_gemm": lib},
        "ffn_block_decode": ffn_block,
        "h_bitlinear": h4,
        "cpu_baseline": cpu,
        "other_workloads": configs,
        "source_digest": digest,
    }
    log("decode step %.2f us (%.1f GB/s); fused decode launch %.3f us avg (%.1f GB/s, %.1f%% of HBM); "
        "two-call step %.2f us; GEMM %.1f us (%.1f TOPS, %.1f%% of int8 peak)" % (
            ms_step * 1e3, value_gbs, fused_us, fused_gbs, 100 * fused_gbs / HBM_PEAK_GBS,
            two_call_us, gemm_us, gemm_tops, 100 * gemm_tops / INT8_PEAK_TOPS))
    log("2:4 prefill GEMM %.1f us (%s)" % (gemm24_us, gemm24_dispatch))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
