"""Single-GPU (MI355X, gfx950) sparse top-k Mixture-of-Experts layer forward.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(``libmoe_mi355x.so``, built in-tree by ``build.py``).  This package is the
thin Python binding: PyTorch supplies device memory and the stream.
"""
from .api import (  # noqa: F401
    MxWeights, Routing, Weights, make_desc, moe_combine, moe_dispatch, moe_experts, moe_forward,
    moe_forward_mx, moe_forward_noalloc, moe_forward_timed,
    moe_grouped_rows,
    moe_resolve_path, moe_route, moe_validate, moe_workspace_size, workspace,
)
from ._lib import MoeDesc, MoeError, lib  # noqa: F401
