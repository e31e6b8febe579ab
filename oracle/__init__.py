"""CPU oracle for the BitLinear forward pass (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports it, and it imports nothing from the product path.

Parity pins: every function here is pinned by `tests/test_oracle_pins.py`
against closed forms, brute force, the pages' printed code mapping and
invariants; no function is "parity unpinned".
"""
from .oracle import (  # noqa: F401
    absmean,
    ternarize,
    nm_keep,
    apply_mask,
    packed_bytes,
    pack_dense,
    pack_nm,
    packed_bytes_trit24,
    pack_trit24,
    unpack_trit24,
    quantize_weights_trit24,
    quantize_weights,
    quant_act,
    quant_act_ex,
    hadamard_rows,
    quant_act_h4,
    quant_act_a48,
    forward,
    forward_a48,
    build,
    LIB_PATH,
)
