"""fp64 CPU oracle for the MiniMind FFN / top-k MoE forward and backward passes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never calls it and
has no CPU fallback.

The oracle shares no code with the HIP path.  It reads the same stored inputs
(bf16/fp32 values widened exactly to float64) and evaluates the method's plain
definition in float64, citing the page passage each step follows.  Every
function is pinned by ``tests/test_oracle_pins.py`` to values the pages print,
closed forms, special cases and brute force; none is "parity unpinned".
"""
from .ffn_moe import (
    silu,
    swiglu_ffn,
    router_probs,
    topk_canonical,
    renorm_weights,
    expert_lists,
    aux_loss,
    moe_route,
    moe_ffn,
    dense_ffn,
    silu_grad,
    swiglu_ffn_bwd,
    moe_ffn_bwd,
    moe_ffn_bwd_sampled,
    logsumexp_rows,
    router_z_loss,
    expert_capacity,
    kept_entries,
)

__all__ = [
    "silu",
    "swiglu_ffn",
    "router_probs",
    "topk_canonical",
    "renorm_weights",
    "expert_lists",
    "aux_loss",
    "moe_route",
    "moe_ffn",
    "dense_ffn",
    "silu_grad",
    "swiglu_ffn_bwd",
    "moe_ffn_bwd",
    "moe_ffn_bwd_sampled",
    "logsumexp_rows",
    "router_z_loss",
    "expert_capacity",
    "kept_entries",
]
