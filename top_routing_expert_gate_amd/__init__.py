"""MI355X-native sparse Mixture-of-Experts FFN forward.

The layer runs in ``libmoe.so`` (hand-written HIP kernels for gfx950 behind
the C ABI of ``include/moe.h``).  ``binding`` mirrors that ABI one function
for one; ``layer.MoELayer`` is a convenience wrapper.  Build the library with
``python -m top_routing_expert_gate_amd.build``.
"""
from .binding import (  # noqa: F401
    MOE_BF16, MOE_EXPERT_SILU_MLP, MOE_EXPERT_SWIGLU, MOE_F32, MOE_SCORE_SIGMOID,
    MOE_SCORE_SOFTMAX, MoeDesc, MoeForwardAux, MoeWeights, lib, make_aux, make_desc,
    make_weights, moe_capacity, moe_check_routing, moe_combine, moe_debug_checks, moe_dispatch, moe_expert_ffn, moe_forward,
    moe_forward_noalloc, moe_route, moe_routed_rows_max, moe_scratch_bytes, moe_status_str,
    moe_workspace_size,
)
