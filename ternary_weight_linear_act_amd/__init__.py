"""BitNet b1.58 BitLinear forward on MI355X (gfx950): packed ternary weights x
int8 activations -> int32 -> fp32, with the Sparse-BitNet N:M variant.

The compute lives in ``libbitlinear.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/bitlinear.h``).  The Python functions below only
marshal torch tensors into that ABI; the library is loaded on first use and a
missing library raises instead of falling back to anything else.
"""
from .binding import (  # noqa: F401
    BitLinearError,
    NM_DENSE,
    NM_2_4,
    NM_6_8,
    packed_size,
    pack_weights,
    pack_weights_masked,
    packed_size_trit24,
    pack_weights_trit24,
    forward_trit24,
    forward_trit24_workspace_size,
    quant_act,
    quant_act_ex,
    quant_act_multi,
    quant_act_h4,
    quant_act_a48,
    combine_a48,
    forward,
    forward_workspace_size,
    forward_noalloc,
    forward_fused,
    forward_grouped,
    forward_grouped_multi,
    forward_fused_ex,
    forward_fused_multi,
    last_dispatch,
    library_path,
    load_library,
)
