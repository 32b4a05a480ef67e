"""GPU parity of the router options against the fp64 oracle: sigmoid scoring
with a selection-only bias, raw (not renormalised) weights, and an expert
capacity that drops the later pairs of an overloaded expert.

Indices, routed counts, the capacity cut (which pairs are dropped, the group
sizes and the grouped order) are compared exactly; weights within 1e-5; y
within the layer tolerance, on both expert-GEMM paths.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_histogram_amd as moe
from cases import Options, custom, make_case
from gpu_util import TOL, check_routing, rel_err, upload
from moe_inputs import NAMED

pytestmark = pytest.mark.gpu

SIG = Options(scoring="sigmoid")
SIG_RAW = Options(scoring="sigmoid", renormalize=False)
RAW = Options(renormalize=False)

# name -> (config, options)
CASES = {
    # DeepSeek-style: sigmoid scores, balancing bias for selection only, one shared expert
    # (sigmoid scores lie in (0, 1), so the bias is kept small enough to mix)
    "sigmoid_bias": (custom("sigmoid_bias", 130, T=200, d=256, E=32, k=4, ffn=128, n_shared=1,
                            ffn_shared=128, bias="normal", bias_var=0.02), SIG),
    "sigmoid_raw": (custom("sigmoid_raw", 131, T=90, d=128, E=16, k=3, ffn=64, bias="normal",
                           bias_var=0.02), SIG_RAW),
    "sigmoid_e256": (custom("sigmoid_e256", 132, T=40, d=256, E=256, k=8, ffn=64,
                            bias="normal", bias_var=0.01), SIG),
    "softmax_raw": (custom("softmax_raw", 133, T=150, d=192, E=16, k=2, ffn=128, bias="normal",
                           bias_var=0.5), RAW),
    "softmax_raw_e128": (custom("softmax_raw_e128", 134, T=33, d=128, E=128, k=4, ffn=64), RAW),
    # skewed load (bias variance 1) so that capacity cuts happen
    "capacity_1": (custom("capacity_1", 135, T=300, d=128, E=8, k=2, ffn=128, bias="normal",
                          bias_var=1.0), Options(capacity_factor=1.0)),
    "capacity_shared": (custom("capacity_shared", 136, T=120, d=192, E=16, k=4, ffn=64,
                               n_shared=1, ffn_shared=64, bias="normal", bias_var=1.0),
                        Options(capacity_factor=0.75)),
    # one token block, router K split: the router's finish kernel runs the capped dispatch
    "capacity_fused": (custom("capacity_fused", 137, T=13, d=512, E=8, k=2, ffn=64,
                              bias="normal", bias_var=1.0), Options(capacity_factor=0.5)),
    # several router blocks, sigmoid scores and a capacity cut together
    "sigmoid_capacity": (custom("sigmoid_capacity", 138, T=260, d=256, E=16, k=2, ffn=64,
                                bias="normal", bias_var=0.02),
                         Options(scoring="sigmoid", capacity_factor=1.25)),
    "f32_sigmoid_capacity": (custom("f32_sigmoid_capacity", 139, T=70, d=64, E=6, k=2, ffn=36,
                                    dtype="f32", bias="normal", bias_var=0.05),
                             Options(scoring="sigmoid", renormalize=False, capacity_factor=0.8)),
    # the wide router form with sigmoid scores and raw weights
    "sigmoid_wide": (custom("sigmoid_wide", 141, T=260, d=4096, E=128, k=4, ffn=64,
                            bias="normal", bias_var=0.02), SIG_RAW),
    # long K: the down GEMM splits K; dropped pairs skip their partial rows too
    "capacity_ksplit": (custom("capacity_ksplit", 140, T=200, d=128, E=3, k=2, ffn=8192,
                               bias="normal", bias_var=1.0), Options(capacity_factor=0.9)),
}


@functools.lru_cache(maxsize=None)
def case_of(name: str):
    cfg, opts = CASES[name]
    return make_case(cfg, opts=opts)


@functools.lru_cache(maxsize=None)
def dev_of(name: str):
    return upload(case_of(name))


@functools.lru_cache(maxsize=None)
def oracle_of(name: str):
    return case_of(name).oracle()


def routing_of(opts: Options) -> moe.Routing:
    return moe.Routing(scoring=opts.scoring, renormalize=opts.renormalize,
                       capacity_factor=opts.capacity_factor or 0.0)


def paths(cfg):
    return ["prefill", "decode"] if cfg.dtype == "bf16" else ["auto"]


def check_capacity_cut(c, ref, slot, offs):
    """slot_row is -1 exactly for the pairs the oracle drops; group sizes are
    the kept counts; kept pairs keep their stable order."""
    cfg = c.cfg
    T, k, E = cfg.T, cfg.k, cfg.E
    keep = ref.keep.ravel()
    slot = slot.ravel()
    assert np.array_equal(slot < 0, ~keep)
    kept_counts = np.bincount(ref.idx.ravel()[keep], minlength=E)
    sizes = np.diff(offs)
    assert np.array_equal(sizes[:E], kept_counts)
    assert np.all(sizes[E:] == T)
    order = oracle.dispatch_order(ref.idx, E)
    order = order[keep[order]]
    exp_slot = np.full(T * k, -1, np.int64)
    exp_slot[order] = np.arange(len(order))
    assert np.array_equal(slot, exp_slot)


@pytest.mark.parametrize("name,path", [(n, p) for n, (cfg, _) in CASES.items()
                                       for p in paths(cfg)])
def test_forward_options(name, path):
    c = case_of(name)
    x, W = dev_of(name)
    ref = oracle_of(name)
    if c.opts.capacity_factor:
        print(f"{name}: capacity {oracle.expert_capacity(c.cfg.T, c.cfg.k, c.cfg.E, c.opts.capacity_factor)}"
              f", dropped {int((~ref.keep).sum())} of {ref.keep.size} pairs")
    y, idx, w, counts = moe.moe_forward(x, W, c.cfg.k, path=path, return_routing=True,
                                        routing=routing_of(c.opts))
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"{name} {path}: max|err|/rms = {err:.3e}")
    assert err <= TOL[c.cfg.dtype], err


@pytest.mark.parametrize("name", list(CASES))
def test_steps_options(name):
    """moe_route with the options, then moe_dispatch with the capacity on the
    oracle's indices, then moe_combine on the oracle's expert outputs."""
    c = case_of(name)
    cfg = c.cfg
    x, W = dev_of(name)
    ref = oracle_of(name)
    T, k, E = cfg.T, cfg.k, cfg.E
    rt = routing_of(c.opts)
    idx, w = moe.moe_route(x, W, k, routing=rt)
    torch.cuda.synchronize()
    check_routing(idx, w, None, ref)

    desc = W.desc(T, k, routing=rt)
    counts, offs, stok, slot = moe.moe_dispatch(
        desc, torch.from_numpy(ref.idx.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    offs = offs.cpu().numpy()
    slot = slot.cpu().numpy()
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    check_capacity_cut(c, ref, slot, offs)
    stok = stok.cpu().numpy()
    kept_rows = offs[E]
    exp_tok = oracle.dispatch_order(ref.idx, E)
    exp_tok = exp_tok[ref.keep.ravel()[exp_tok]] // k
    assert np.array_equal(stok[:kept_rows], exp_tok)
    for s in range(cfg.n_shared):
        assert np.array_equal(stok[offs[E + s]:offs[E + s + 1]], np.arange(T))

    # combine on exact expert outputs of the kept rows
    X = oracle.widen(c.x, cfg.dtype)
    R = moe.moe_grouped_rows(desc)
    out = np.zeros((R, cfg.d))
    for g in range(E + cfg.n_shared):
        r0, r1 = offs[g], offs[g + 1]
        if r1 > r0:
            ws = c.expert(g) if g < E else c.shared(g - E)
            out[r0:r1] = oracle.swiglu_expert(X[stok[r0:r1]],
                                              *(oracle.widen(a, cfg.dtype) for a in ws))
    y = moe.moe_combine(desc, torch.from_numpy(out.astype(np.float32)).cuda(),
                        torch.from_numpy(ref.w.astype(np.float32)).cuda(),
                        torch.from_numpy(slot.astype(np.int32).reshape(T, k)).cuda(),
                        torch.from_numpy(offs.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), ref.y) <= 1e-5


@pytest.mark.parametrize("extra", [0, 1000])
def test_capacity_without_drops_is_dropless(extra):
    """A capacity at or above the busiest expert's count (the cut runs but
    drops nothing), or above T pairs (no cut): the output equals the
    dropless layer's bit for bit."""
    c = case_of("capacity_1")
    x, W = dev_of("capacity_1")
    cfg = c.cfg
    busiest = int(oracle_of("capacity_1").counts.max())
    factor = (busiest + extra) * cfg.E / (cfg.T * cfg.k)
    cap = oracle.expert_capacity(cfg.T, cfg.k, cfg.E, factor)
    assert busiest <= cap and (extra > 0 or cap < cfg.T)
    a = moe.moe_forward(x, W, cfg.k, return_routing=True)
    b = moe.moe_forward(x, W, cfg.k, return_routing=True,
                        routing=moe.Routing(capacity_factor=factor))
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_sigmoid_without_bias_selects_by_logit():
    """Sigmoid is increasing, so without a bias the sigmoid router keeps the
    same experts in the same order as the softmax router."""
    c = case_of("softmax_raw_e128")  # no bias
    x, W = dev_of("softmax_raw_e128")
    i1, _ = moe.moe_route(x, W, c.cfg.k)
    i2, w2 = moe.moe_route(x, W, c.cfg.k, routing=moe.Routing(scoring="sigmoid"))
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert float((w2.sum(dim=1) - 1).abs().max()) < 1e-6


@pytest.mark.parametrize("T", [4096])
def test_deepseek_sigmoid_full_size(T):
    """The DeepSeek-V3-shaped layer (256 experts, top-8, one shared expert,
    bias ~ N(0, 0.5)) with sigmoid scores and the bias steering selection
    only: routing, counts and y on every token."""
    cfg = NAMED["deepseek_v3"]
    c = make_case(cfg, T, opts=SIG)
    x, W = upload(c)
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward(x, W, cfg.k, return_routing=True,
                                        routing=moe.Routing(scoring="sigmoid"))
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"deepseek_v3 sigmoid T={T}: max|err|/rms = {err:.3e}, "
          f"experts touched {int((counts > 0).sum())}")
    assert err <= TOL[cfg.dtype], err
