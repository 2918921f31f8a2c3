"""CPU oracle for the routed-expert W4A16 group-32 MoE layer.

Test infrastructure only: imported by ``tests/``, by the smoke check in
``__graft_entry__.py`` and by the CPU-baseline leg of ``bench.py``.  It shares
no code with the HIP library and never imports it.
"""

from .moe_oracle import (  # noqa: F401
    GROUP_SIZE,
    block,
    combine,
    dequantize,
    expert_ffn,
    grouped_ffn,
    layer,
    layer_with_shared,
    permute,
    route,
    router_logits,
    shared_expert,
    silu,
    token_outputs,
    unpack_weight_codes,
    unpack_zero_codes,
)
