"""The forward pass allocates nothing, synchronises nothing and launches only
on the caller's stream, so it runs on any stream and can be captured in a
HIP graph (torch.cuda.graph) and replayed with new token values: routing,
grouping and tile schedules are rebuilt on the device at every replay.

Each replay is checked, bit for bit, against an eager call on the same
inputs (the layer is deterministic), with unrelated eager work and a device
synchronisation between replays; eager results are themselves held to the
fp64 oracle by the parity tests.
"""
from __future__ import annotations

import pytest
import torch

import sparse_mixture_experts_histogram_amd as moe
from cases import custom, make_case
from gpu_util import TOL, check_routing, rel_err, upload

pytestmark = pytest.mark.gpu

CASES = {
    # 600 tokens x top-2 over 16 experts (128-row prefill tiles), a shared
    # expert with a different ffn, and a selection bias
    "prefill_shared": (custom("graph_prefill", 170, T=600, d=256, E=16, k=2, ffn=192,
                              n_shared=1, ffn_shared=320, bias="normal", bias_var=0.5),
                       "prefill"),
    "decode": (custom("graph_decode", 171, T=8, d=512, E=32, k=4, ffn=256), "decode"),
    "f32": (custom("graph_f32", 172, T=100, d=64, E=8, k=2, ffn=96, dtype="f32"), "auto"),
}


def _variants(x: torch.Tensor, n: int):
    """n token batches of x's shape: row permutations and sign flips of x
    (each changes which experts the tokens pick, and so the group sizes)."""
    g = torch.Generator(device="cpu").manual_seed(5)
    out = []
    for i in range(n):
        perm = torch.randperm(x.shape[0], generator=g).to(x.device)
        v = x[perm]
        out.append(-v if i % 2 else v)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay(name):
    cfg, path = CASES[name]
    c = make_case(cfg)
    x, W = upload(c)
    ref = c.oracle()
    ws = moe.workspace(W.desc(cfg.T, cfg.k, torch.float32, path), x.device)
    xs = x.clone()
    # warm-up on a side stream, as torch's graph capture expects
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward(xs, W, cfg.k, path=path, ws=ws, return_routing=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = moe.moe_forward(xs, W, cfg.k, path=path, ws=ws, return_routing=True)
    torch.cuda.synchronize()

    # first replay on the case's own tokens: against the oracle
    graph.replay()
    torch.cuda.synchronize()
    check_routing(outs[1], outs[2], outs[3], ref)
    assert rel_err(outs[0].cpu().numpy(), ref.y) <= TOL[cfg.dtype]

    ws_eager = torch.empty_like(ws)
    for v in _variants(x, 4):
        xs.copy_(v)
        noise = torch.randn(1 << 20, device=x.device).sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = moe.moe_forward(v, W, cfg.k, path=path, ws=ws_eager, return_routing=True)
        torch.cuda.synchronize()
        for got, exp in zip(outs, want):
            assert torch.equal(got, exp)
        assert torch.isfinite(noise)


def test_side_stream():
    """The same call on a non-default stream gives the same bits."""
    cfg, path = CASES["prefill_shared"]
    c = make_case(cfg)
    x, W = upload(c)
    a = moe.moe_forward(x, W, cfg.k, path=path, return_routing=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = moe.moe_forward(x, W, cfg.k, path=path, return_routing=True)
    s.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_graph_replay_mx(fmt):
    """The MX-format forward (LDS-staged kernel: at least one pair per
    expert) under graph capture and replay."""
    from test_gpu_mxfp4 import MxCase
    cfg = custom(f"graph_{fmt}", 173, T=64, d=256, E=8, k=2, ffn=192)
    c = MxCase(cfg, fmt=fmt)
    x, W = c.upload()
    ref = c.oracle()
    ws = moe.workspace(W.desc(cfg.T, cfg.k), x.device)
    xs = x.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward_mx(xs, W, cfg.k, ws=ws, return_routing=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = moe.moe_forward_mx(xs, W, cfg.k, ws=ws, return_routing=True)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    check_routing(outs[1], outs[2], outs[3], ref)
    assert rel_err(outs[0].cpu().numpy(), ref.y) <= TOL["bf16"]
    ws_eager = torch.empty_like(ws)
    for v in _variants(x, 3):
        xs.copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = moe.moe_forward_mx(v, W, cfg.k, ws=ws_eager, return_routing=True)
        torch.cuda.synchronize()
        for got, exp in zip(outs, want):
            assert torch.equal(got, exp)
