"""Build libbitlinear.so (hand-written HIP for gfx950) in-tree with hipcc.

Each .hip source compiles to an object under _build/ in parallel, then one
link step writes ternary_weight_linear_act_amd/libbitlinear.so.  Flags:
gfx950 only; -ffp-contract=off and IEEE-rounded fp32 division so the
quantisation decisions match their written definition; packed-fp32 VALU
instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
SOURCES = ["api.hip", "quant.hip", "pack.hip", "gemv.hip", "gemm.hip", "gemm_sparse.hip", "skinny.hip", "skinny_direct.hip", "skinny_direct_tiles.hip", "trit24.hip", "fused.hip", "decode_dot4.hip",
           "decode_dot4_tr.hip", "decode_multi.hip", "noalloc.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-pass-failed",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "probe", "libstreamprobe.so")


def build_probe(verbose: bool = True) -> str:
    """The streaming-read probe bench.py's --stream-probe leg loads (not part
    of the BitLinear path)."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *CFLAGS, "-shared", "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL if not verbose else None)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if out and verbose:
            print(out, flush=True)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: %s" % ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
