"""CPU check of the fast N:M decode used by the forward kernels.

tests/host/nm_decode_check.cpp includes the kernels' common header as host
code and, on 200000 random valid superblocks per pattern, compares
decode_superblock_fast (transpose + table / insertion) with the bit-by-bit
decode_superblock, and the one-token permute dot (nm_dot_superblock, with
v_perm_b32 and v_dot4 emulated) with sum (c - 1) * x over the reference
decode on random int8 activations.  The GPU parity tests then check the
kernels against the oracle.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_fast_nm_decode_matches_reference(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = str(tmp_path / "nm_decode_check")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "ternary_weight_linear_act_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host", "nm_decode_check.cpp"),
                    "-o", exe], check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches 2:4 0 6:8 0" in out.stdout
