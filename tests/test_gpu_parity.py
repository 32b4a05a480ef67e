"""GPU parity: every step and the whole layer through the C ABI, against the
fp64 oracle on the same seeded inputs.

Small layers cover several tiles and ragged tails of every kernel; the named
layers run at their full sizes, with routing, counts and outputs checked on
every token.  Both expert-GEMM paths (prefill and decode kernels) are
checked on the same inputs.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_histogram_amd as moe
from cases import Case, custom, make_case
from gpu_util import TOL, check_routing, rel_err, upload
from moe_inputs import NAMED

pytestmark = pytest.mark.gpu

SMALL = {c.name: c for c in [
    custom("ragged_t300", 101, T=300, d=256, E=8, k=2, ffn=320),
    custom("shared2", 102, T=77, d=192, E=16, k=4, ffn=128, n_shared=2, ffn_shared=192),
    custom("bias_e32", 103, T=130, d=128, E=32, k=3, ffn=64, bias="normal", bias_var=0.5),
    custom("top1", 104, T=50, d=64, E=4, k=1, ffn=64),
    custom("one_expert", 105, T=33, d=128, E=1, k=1, ffn=128),
    custom("k_equals_e", 106, T=40, d=128, E=4, k=4, ffn=64),
    custom("e256_k8_shared", 107, T=64, d=256, E=256, k=8, ffn=128, n_shared=1, ffn_shared=128,
           bias="normal", bias_var=0.5),
    custom("e512_k32", 108, T=20, d=64, E=512, k=32, ffn=64),
    custom("f32_ragged", 109, T=45, d=96, E=6, k=2, ffn=40, dtype="f32"),
    custom("f32_shared", 110, T=70, d=64, E=5, k=3, ffn=36, n_shared=1, ffn_shared=52,
           dtype="f32"),
    custom("one_token", 111, T=1, d=128, E=8, k=2, ffn=128),
    # >= 384 rows per expert: the 256-row prefill tiles, ragged last tiles
    custom("rows256", 112, T=900, d=192, E=2, k=1, ffn=320),
    # long K and few tiles: the down GEMM splits K in two (partials summed in the combine)
    custom("ksplit", 113, T=200, d=128, E=3, k=2, ffn=8192),
    # one token block, router K split over workgroups: the router's finish kernel runs
    # the dispatch itself (with a shared expert and a logit bias)
    custom("fused_dispatch", 114, T=13, d=512, E=64, k=6, ffn=128, n_shared=1, ffn_shared=192,
           bias="normal", bias_var=0.5),
    # several token blocks with the router K split over workgroups, two shared experts
    custom("split_router", 115, T=100, d=512, E=16, k=2, ffn=64, n_shared=2, ffn_shared=64),
    # many tokens and a large router matrix (E * d >= 2^19): the wide router
    # (64-token workgroups over K parts); T not a multiple of 64
    custom("wide_router", 116, T=300, d=4096, E=128, k=4, ffn=64, bias="normal", bias_var=0.5),
    # 128-row prefill tiles with skewed loads (two experts over 500 rows,
    # one with 2) and a shared expert of 1200 rows
    custom("split_tiles", 117, T=1200, d=256, E=16, k=2, ffn=192, n_shared=1, ffn_shared=320,
           bias="normal", bias_var=0.5),
    # a down GEMM of 256-row tiles with K >= 8192 whose last round is split
    # along K into pieces added by the fixup kernel (4 tiles on 256 slots:
    # 16 pieces of 8 slabs each)
    custom("last_round", 118, T=800, d=256, E=2, k=1, ffn=8192),
    # the same with a shared expert whose reduction is longer than the
    # routed experts' (pieces of unequal length), 16 tiles of 16 pieces
    custom("last_round_shared", 119, T=800, d=512, E=2, k=1, ffn=8192, n_shared=1,
           ffn_shared=8448, bias="normal", bias_var=0.5),
    # the all-rows 256-row down form (experts of 128 to 384 rows: 300 each)
    # with K >= 8192: 4 tiles of 16 pieces, added by the fixup's 8-wave form
    custom("last_round_all_rows", 121, T=600, d=256, E=2, k=1, ffn=8192),
    NAMED["tiny_f32"],
]}


@functools.lru_cache(maxsize=None)
def case_of(name: str, T: int = -1) -> Case:
    cfg = SMALL.get(name) or NAMED[name]
    return make_case(cfg, None if T < 0 else T)


@functools.lru_cache(maxsize=None)
def dev_of(name: str, T: int = -1):
    return upload(case_of(name, T))


@functools.lru_cache(maxsize=None)
def oracle_of(name: str, T: int = -1):
    return case_of(name, T).oracle()


def paths(cfg):
    return ["prefill", "decode"] if cfg.dtype == "bf16" else ["auto"]


SMALL_PATHS = [(n, p) for n, c in SMALL.items() for p in paths(c)]


@pytest.mark.parametrize("name,path", SMALL_PATHS)
def test_forward_small(name, path):
    c = case_of(name)
    x, W = dev_of(name)
    ref = oracle_of(name)
    y, idx, w, counts = moe.moe_forward(x, W, c.cfg.k, path=path, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"{name} {path}: max|err|/rms = {err:.3e}")
    assert err <= TOL[c.cfg.dtype], err


@pytest.mark.parametrize("name", list(SMALL))
def test_steps_small(name):
    """moe_route, moe_dispatch, moe_experts, moe_combine one by one; each
    later step is fed the oracle's result of the earlier ones."""
    c = case_of(name)
    cfg = c.cfg
    x, W = dev_of(name)
    ref = oracle_of(name)
    T, k, E = cfg.T, cfg.k, cfg.E
    idx, w = moe.moe_route(x, W, k)
    torch.cuda.synchronize()
    check_routing(idx, w, None, ref)

    # dispatch on the oracle's indices
    desc = W.desc(T, k)
    idx_ref = torch.from_numpy(ref.idx.astype(np.int32)).cuda()
    counts, offs, stok, slot = moe.moe_dispatch(desc, idx_ref)
    order = oracle.dispatch_order(ref.idx, E)
    exp_counts = ref.counts
    exp_offs = np.concatenate([[0], np.cumsum(np.concatenate(
        [exp_counts, np.full(cfg.n_shared, T)]))]).astype(np.int32)
    exp_stok = np.concatenate([order // k] + [np.arange(T)] * cfg.n_shared).astype(np.int32)
    exp_slot = np.empty(T * k, np.int32)
    exp_slot[order] = np.arange(T * k)
    assert np.array_equal(counts.cpu().numpy(), exp_counts)
    assert np.array_equal(offs.cpu().numpy(), exp_offs)
    assert np.array_equal(stok.cpu().numpy(), exp_stok)
    assert np.array_equal(slot.cpu().numpy().ravel(), exp_slot)

    # experts on the oracle's grouping.  For bf16 layers the kernels round h
    # to bf16 (half an ulp: 2^-9 relative) before the down GEMM, so each
    # expert output may differ from the fp64 value by up to
    # 2^-9 * sum_j |h_j| |W_down[:, j]|; the check allows twice that (fp32
    # accumulation adds far less) on every element.  (The layer output y,
    # checked above and below, keeps the rms bar.)
    X = oracle.widen(c.x, cfg.dtype)
    exp_out = bound = None
    for path in paths(cfg):
        out = moe.moe_experts(x, W, k, torch.from_numpy(exp_offs).cuda(),
                              torch.from_numpy(exp_stok).cuda(), path=path)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        if exp_out is None:
            exp_out = np.zeros_like(out, dtype=np.float64)
            bound = np.zeros_like(exp_out)
            for g in range(E + cfg.n_shared):
                r0, r1 = exp_offs[g], exp_offs[g + 1]
                if r1 == r0:
                    continue
                wu, wg, wd = (oracle.widen(a, cfg.dtype)
                              for a in (c.expert(g) if g < E else c.shared(g - E)))
                Xg = X[exp_stok[r0:r1]]
                exp_out[r0:r1] = oracle.swiglu_expert(Xg, wu, wg, wd)
                H = oracle.silu(Xg @ wg.T) * (Xg @ wu.T)
                bound[r0:r1] = 2.0 ** -8 * (np.abs(H) @ np.abs(wd).T)
        err = rel_err(out, exp_out)
        if cfg.dtype == "bf16":
            excess = np.abs(out.astype(np.float64) - exp_out) - bound
            assert excess.max() <= 1e-6 * np.sqrt(np.mean(exp_out ** 2)), (path, excess.max())
        else:
            assert err <= TOL[cfg.dtype], (path, err)

    # combine on the oracle's expert outputs and weights
    out_ref = torch.from_numpy(exp_out.astype(np.float32)).cuda()
    y = moe.moe_combine(desc, out_ref, torch.from_numpy(ref.w.astype(np.float32)).cuda(),
                        torch.from_numpy(exp_slot.reshape(T, k)).cuda(),
                        torch.from_numpy(exp_offs).cuda())
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), ref.y) <= 1e-5


def test_zero_tokens():
    c = case_of("ragged_t300")
    x, W = dev_of("ragged_t300")
    y, idx, w, counts = moe.moe_forward(x[:0], W, c.cfg.k, return_routing=True)
    torch.cuda.synchronize()
    assert y.shape == (0, c.cfg.d) and idx.shape == (0, c.cfg.k)


@pytest.mark.parametrize("k", [4, 2])
def test_all_ties_mean_of_experts(k):
    """Zero router weights: every logit ties, so top-k is experts 0..k-1 with
    weight 1/k each and y is the mean of those experts (k = E: all experts)."""
    cfg = custom("ties", 120, T=24, d=128, E=4, k=k, ffn=64, margin=0.0)
    c = make_case(cfg)
    c.w_router = np.zeros_like(c.w_router)
    ref = c.oracle()
    assert np.all(ref.idx == np.arange(k))
    x, W = upload(c)
    for path in ("prefill", "decode"):
        y, idx, w, counts = moe.moe_forward(x, W, k, path=path, return_routing=True)
        torch.cuda.synchronize()
        assert np.all(idx.cpu().numpy() == np.arange(k))
        assert np.all(w.cpu().numpy() == np.float32(1.0 / k))
        assert rel_err(y.cpu().numpy(), ref.y) <= TOL["bf16"]


def test_deterministic():
    c = case_of("e256_k8_shared")
    x, W = dev_of("e256_k8_shared")
    a = moe.moe_forward(x, W, c.cfg.k, return_routing=True)
    b = moe.moe_forward(x, W, c.cfg.k, return_routing=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_bf16_output():
    c = case_of("ragged_t300")
    x, W = dev_of("ragged_t300")
    ref = oracle_of("ragged_t300")
    y = moe.moe_forward(x, W, c.cfg.k, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    err = rel_err(y.float().cpu().numpy(), ref.y)
    print(f"bf16 y: max|err|/rms = {err:.3e}")
    assert err <= 2 * TOL["bf16"]


# ------------------------------------------------------------------ full-size layers
FULL = [("mixtral", 4096), ("mixtral", 16), ("midsize_zipf", 8192), ("gpt_oss", 1),
        ("gpt_oss", 8), ("gpt_oss", 32), ("gpt_oss", 128), ("gpt_oss", 512),
        ("deepseek_v3", 4096)]


@pytest.mark.parametrize("name,T", FULL)
def test_forward_full_size(name, T):
    """Routing and counts bit-exact and y within tolerance, on every token, in
    the launch configuration the benchmark uses (AUTO path)."""
    c = case_of(name, T)
    x, W = dev_of(name, T)
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward(x, W, c.cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    touched = int((counts > 0).sum())
    print(f"{name} T={T} path={moe.moe_resolve_path(W.desc(T, c.cfg.k))}: "
          f"max|err|/rms = {err:.3e}, experts touched {touched}")
    assert err <= TOL[c.cfg.dtype], err
