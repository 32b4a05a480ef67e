"""fp64 CPU oracle of the sparse top-k MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the package smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the GPU path;
both read the same seeded inputs from ``moe_inputs``.

Every function is plain numpy in float64 and follows the steps the source
pages give for one MoE layer (see the docstrings of ``oracle.moe``).
"""
from .moe import (  # noqa: F401
    widen, router_logits, softmax, select_topk, renormalise, route, expert_counts,
    dispatch_order, silu, swiglu_expert, moe_forward, topk_gaps, share_touched,
    sigmoid, kept_scores, selection_keys, expert_capacity, capacity_keep, e2m1_value,
    e8m0_value, dequant_mxfp4, e4m3_value, dequant_mxfp8, widen_weight, MoEResult,
)
