"""Seeded synthetic inputs for the BitLinear workloads.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic (no quantisation, no packing, no contraction), so both the
CPU oracle's tests and the HIP path can take their inputs from it.

Recipe: numpy ``default_rng(seed)`` float64 standard normals, scaled, then cast
to float32.  Within a workload the weight matrices are drawn first, in the
order listed, then the activations, in the order listed.  Latent weights are
N(0, 0.02^2) (the BitLinear initialisation in "BitNet 논문 분석: 1-Bit LLM의
시대", section "Absmean 양자화 함수"); activations are N(0, 1), optionally with
a fraction of entries multiplied by an outlier factor.  The model shapes
(2B-class FFN, Qwen2.5-1.5B-like FFN, 3B-class block) are synthetic stand-ins:
no page prints them and no trained weights are used.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_SIGMA = 0.02


@dataclass(frozen=True)
class Proj:
    """One BitLinear projection: K inputs -> N outputs, with an N:M pattern."""
    name: str
    K: int
    N: int
    nm: tuple = (0, 0)          # (0, 0) dense, (2, 4), (6, 8)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    projs: tuple                 # tuple[Proj]
    Ms: tuple                    # token counts
    outlier_frac: float = 0.0    # fraction of activation entries scaled by outlier_mul
    outlier_mul: float = 20.0
    notes: str = ""
    groups: tuple = ()           # projections that read the same activations (q/k/v, gate/up)


WORKLOADS = {
    # single BitLinear 1024 -> 1024, M in {1, 16}
    "single_1024": Workload(
        "single_1024", 0, (Proj("linear", 1024, 1024),), (1, 16),
        notes="single BitLinear K=N=1024, small enough for the oracle in seconds"),
    # 2B-class FFN decode, M = 1: gate/up 2560 -> 6912 and down 6912 -> 2560
    "decode_ffn_2b": Workload(
        "decode_ffn_2b", 1,
        (Proj("gate", 2560, 6912), Proj("up", 2560, 6912), Proj("down", 6912, 2560)),
        (1,), outlier_frac=0.001,
        notes="decode GEMV at 2B-class FFN shapes, 0.1% activation outliers x20",
        groups=(("gate", "up"), ("down",))),
    # prefill GEMM M = 2048, K = 2560, N = 6912
    "prefill_2048": Workload(
        "prefill_2048", 2, (Proj("up", 2560, 6912),), (2048,),
        notes="prefill GEMM M=2048 K=2560 N=6912"),
    # Sparse-BitNet N:M at Qwen2.5-1.5B-like FFN 1536 -> 8960, M in {1, 512}
    "sparse_ffn_1p5b": Workload(
        "sparse_ffn_1p5b", 3,
        (Proj("dense", 1536, 8960, (0, 0)), Proj("nm24", 1536, 8960, (2, 4)),
         Proj("nm68", 1536, 8960, (6, 8))),
        (1, 512),
        notes="N:M variants 2:4 and 6:8 vs dense, K=1536 N=8960"),
    # 3B-class block: q,k,v,o, gate, up, down, M in {1, 8, 64}
    "block_3b": Workload(
        "block_3b", 4,
        (Proj("q", 2048, 2048), Proj("k", 2048, 256), Proj("v", 2048, 256),
         Proj("o", 2048, 2048), Proj("gate", 2048, 11008), Proj("up", 2048, 11008),
         Proj("down", 11008, 2048)),
        (1, 8, 64),
        notes="batched decode sweep over the seven projections of one 3B-class block",
        groups=(("q", "k", "v"), ("o",), ("gate", "up"), ("down",))),
}


def normal_f32(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


def activations(rng: np.random.Generator, M: int, K: int, outlier_frac: float = 0.0,
                outlier_mul: float = 20.0) -> np.ndarray:
    """M x K N(0,1) fp32; max(1, round(frac*M*K)) distinct entries multiplied by outlier_mul."""
    X = rng.standard_normal((M, K))
    if outlier_frac > 0 and M * K > 0:
        cnt = max(1, int(round(outlier_frac * M * K)))
        idx = rng.choice(M * K, size=cnt, replace=False)
        X.reshape(-1)[idx] *= outlier_mul
    return X.astype(np.float32)


@dataclass
class Drawn:
    workload: Workload
    W: dict = field(default_factory=dict)     # proj name -> N x K fp32
    X: dict = field(default_factory=dict)     # (proj name, M) -> M x K fp32


def input_groups(wl: Workload):
    """Groups of projections sharing one activation input, in listed order."""
    if wl.groups:
        return [tuple(g) for g in wl.groups]
    return [(p.name,) for p in wl.projs]


def draw(name: str, projs=None, Ms=None) -> Drawn:
    """Draw every weight (in listed order), then one activation matrix per
    input group and token count (group-major, then M).  Projections of a group
    (q/k/v, gate/up) share the same activation array.

    ``projs``/``Ms`` restrict what is returned, but the generator still walks the
    full order so a subset gets the same values as the full draw.
    """
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    out = Drawn(wl)
    for p in wl.projs:
        w = normal_f32(rng, (p.N, p.K), WEIGHT_SIGMA)
        if projs is None or p.name in projs:
            out.W[p.name] = w
    K_of = {p.name: p.K for p in wl.projs}
    for group in input_groups(wl):
        K = K_of[group[0]]
        for M in wl.Ms:
            x = activations(rng, M, K, wl.outlier_frac, wl.outlier_mul)
            for pname in group:
                if (projs is None or pname in projs) and (Ms is None or M in Ms):
                    out.X[(pname, M)] = x
    return out


def small_case(seed: int, M: int, N: int, K: int, outlier_frac: float = 0.0):
    """An ad-hoc seeded case (ragged shapes, edge cases): returns (W, X)."""
    rng = np.random.default_rng(seed)
    W = normal_f32(rng, (N, K), WEIGHT_SIGMA)
    X = activations(rng, M, K, outlier_frac)
    return W, X
