"""The no-allocation entry point (moe_forward_noalloc, scratch held inside
the library per GPU) against moe_forward with a caller workspace: the same
kernels on the same inputs, so routing and y must be bit-identical, and y
within the layer tolerance of the fp64 oracle.  Two calls in a row, the
second with fewer tokens (and the other expert-GEMM path), so the second
runs on scratch that still holds the first call's contents."""
from __future__ import annotations

import pytest
import torch

import sparse_mixture_experts_histogram_amd as moe
from cases import custom, make_case
from gpu_util import TOL, check_routing, rel_err, upload

pytestmark = pytest.mark.gpu


def _both(x, W, k):
    a = moe.moe_forward(x, W, k, return_routing=True)
    b = moe.moe_forward_noalloc(x, W, k, return_routing=True)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_matches_workspace_entry_point():
    cfg = custom("noalloc", 170, T=300, d=512, E=16, k=4, ffn=256, n_shared=1, ffn_shared=128,
                 bias="normal", bias_var=0.5)
    c = make_case(cfg)
    x, W = upload(c)
    ref = c.oracle()
    for T, path in ((300, "prefill"), (20, "decode")):
        xt = x[:T].contiguous()
        assert moe.moe_resolve_path(W.desc(T, cfg.k)) == path
        a, b = _both(xt, W, cfg.k)
        for u, v, name in zip(a, b, ("y", "idx", "w", "counts")):
            assert torch.equal(u, v), (T, name)
        if T == cfg.T:
            check_routing(b[1], b[2], b[3], ref)
            err = rel_err(b[0].cpu().numpy(), ref.y)
            print(f"noalloc T={T}: bit-identical to moe_forward; max|err|/rms = {err:.3e}")
            assert err <= TOL["bf16"], err
        else:
            print(f"noalloc T={T} ({path}): bit-identical to moe_forward")


def test_noalloc_rejects_large_layer():
    """A layer needing more than the library's scratch is refused before any
    launch, with MOE_ERR_TOO_LARGE."""
    cfg = custom("noalloc_big", 171, T=2048, d=1024, E=4, k=2, ffn=8192)
    c = make_case(cfg)
    x, W = upload(c)
    assert moe.moe_workspace_size(W.desc(cfg.T, cfg.k)) > moe._lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError, match="MOE_ERR_TOO_LARGE"):
        moe.moe_forward_noalloc(x, W, cfg.k)
