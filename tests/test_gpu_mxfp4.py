"""GPU parity of layers whose expert weights are MXFP4 (packed E2M1 codes with
one E8M0 scale per 32 elements along K) against the fp64 oracle, which
dequantises them from the format's definition.

Indices and counts exact, weights within 1e-5, y within the bf16 layer
tolerance: the dequantised weights are bf16 values, so the products are the
same exact bf16 products as in a bf16 layer.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import sparse_mixture_experts_histogram_amd as moe
from cases import custom, margin_x
from gpu_util import TOL, check_routing, h_rounding_bound, rel_err, to_dev
from moe_inputs import NAMED, generate, tables

pytestmark = pytest.mark.gpu

# Two kernels run MXFP4 experts: the direct-load one (fewer (token, expert)
# pairs than a quarter of the experts, or K above 3072) and the LDS-staged one
# (16 x 128 up/gate tiles, 16 x 64 down tiles, K in stages of 256 through a
# 3-slot ring).  mx_few_pairs and the gpt-oss T=1 layer take the first;
# mx_long_k takes it for up/gate only; the rest take the second: mx_ragged
# and mx_shared with partial 128-feature tiles, mx_stages with 5 and 4
# stages (the ring's two tail forms), mx_k2880 with a last stage of 2 blocks.
# In the direct-load kernel K = 2880 (45 units of 64) splits over four waves
# in ranges that are not multiples of its load batch.
SMALL = {c.name: c for c in [
    custom("mx_ragged", 150, T=150, d=256, E=8, k=2, ffn=192),
    custom("mx_shared", 151, T=70, d=128, E=16, k=4, ffn=64, n_shared=1, ffn_shared=128,
           bias="normal", bias_var=0.5),
    custom("mx_one_token", 152, T=1, d=192, E=8, k=2, ffn=128),
    custom("mx_k_equals_e", 153, T=33, d=64, E=4, k=4, ffn=64),
    custom("mx_k2880", 154, T=40, d=2880, E=4, k=2, ffn=2880),
    custom("mx_stages", 155, T=64, d=1280, E=8, k=2, ffn=1024),
    custom("mx_long_k", 156, T=24, d=4096, E=4, k=2, ffn=128),
    custom("mx_few_pairs", 157, T=3, d=2880, E=32, k=2, ffn=384),
]}


class MxCase:
    def __init__(self, cfg, T=None, x=None, fmt="mxfp4"):
        self.cfg = cfg
        self.fmt = fmt
        T = cfg.T if T is None else T
        self.w_router = generate.router_weight(cfg)
        self.bias = generate.normal_bias(cfg) if cfg.bias == "normal" else None
        self.x = x if x is not None else margin_x(cfg, T, self.w_router, self.bias)
        stack = generate.stacked_mxfp4 if fmt == "mxfp4" else generate.stacked_mxfp8
        self.mx = stack(cfg)
        self.smx = stack(cfg, shared=True) if cfg.n_shared else None

    def expert(self, e):
        u, us, g, gs, d, ds = self.mx
        return (u[e], us[e]), (g[e], gs[e]), (d[e], ds[e])

    def shared(self, s):
        u, us, g, gs, d, ds = self.smx
        return (u[s], us[s]), (g[s], gs[s]), (d[s], ds[s])

    def oracle(self, tokens=None):
        import oracle
        c = self.cfg
        return oracle.moe_forward(self.x, self.w_router, self.bias, c.k, self.expert, c.E, "bf16",
                                  self.shared if c.n_shared else None, c.n_shared, tokens,
                                  expert_dtype=self.fmt)

    def upload(self, line_rows=False):
        """Device tensors of the layer.  line_rows: code rows padded to whole
        128-byte lines (MOE_FLAG_MX_LINE_ROWS), the padding filled with 0xFF
        bytes (NaN codes in E4M3, -6 in E2M1: a kernel reading them would
        change y)."""
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        tc = (lambda a: t(pad_rows(a))) if line_rows else t
        u, us, g, gs, d, ds = self.mx
        W = moe.MxWeights(w_router=to_dev(self.w_router, "bf16"), up=tc(u), up_scale=t(us),
                          gate=tc(g), gate_scale=t(gs), down=tc(d), down_scale=t(ds),
                          bias=None if self.bias is None else t(self.bias),
                          line_rows=line_rows, expert_format=self.fmt)
        if self.smx is not None:
            su, sus, sg, sgs, sd, sds = self.smx
            W.s_up, W.s_up_scale, W.s_gate, W.s_gate_scale = tc(su), t(sus), tc(sg), t(sgs)
            W.s_down, W.s_down_scale = tc(sd), t(sds)
        return to_dev(self.x, "bf16"), W


def pad_rows(a: np.ndarray) -> np.ndarray:
    """Code rows (last axis) padded with 0xFF bytes to a multiple of 128."""
    R = a.shape[-1]
    out = np.full(a.shape[:-1] + ((R + 127) // 128 * 128,), 0xFF, dtype=np.uint8)
    out[..., :R] = a
    return out


@functools.lru_cache(maxsize=None)
def case_of(name):
    return MxCase(SMALL[name])


@pytest.mark.parametrize("name", list(SMALL))
def test_mxfp4_small(name):
    c = case_of(name)
    x, W = c.upload()
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward_mx(x, W, c.cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"{name}: max|err|/rms = {err:.3e}")
    assert err <= TOL["bf16"], err


def test_mxfp4_rejects_dense_entry_points():
    """A descriptor with MXFP4 experts is refused by moe_forward and
    moe_experts, and a dense one by moe_forward_mx."""
    c = case_of("mx_ragged")
    x, W = c.upload()
    desc = W.desc(c.cfg.T, c.cfg.k)
    L = moe.lib()
    assert L.moe_forward(desc, None, None, None, None, None, None, None, None, None, None, None,
                         None, None, None, 0, None) == -1
    dense = moe.make_desc(c.cfg.T, c.cfg.d, c.cfg.E, c.cfg.k, c.cfg.ffn)
    sc = moe._lib.MoeMxScales()
    assert L.moe_forward_mx(dense, None, None, None, None, None, None, None, None, None, sc, None,
                            None, None, None, None, 0, None, None) == -1


@pytest.mark.parametrize("T", [1, 8, 32, 128, 512])
def test_mxfp4_gpt_oss_full_size(T):
    """The gpt-oss-shaped layer (d=2880, 128 experts, top-4) with MXFP4
    experts at decode batch sizes: routing and y on every token (T = 32 is
    the first batch with as many pairs as experts, where the LDS-staged
    kernel takes over)."""
    cfg = NAMED["gpt_oss"]
    li = tables.layer_inputs(cfg, T)
    c = MxCase(cfg, T, x=li.x)
    x, W = c.upload()
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward_mx(x, W, cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"gpt_oss mxfp4 T={T}: max|err|/rms = {err:.3e}, touched {int((counts > 0).sum())}")
    assert err <= TOL["bf16"], err


# MXFP8 (E4M3 codes, one per byte): the LDS-staged kernel at every batch
# size, 16 x 64 tiles with 4 waves; stage tails (K = 1280: 5 stages, 1024: 4),
# partial tiles (ffn = 192), a shared expert, a single token, long K (4096).
SMALL8 = {c.name: c for c in [
    custom("mx8_ragged", 160, T=150, d=256, E=8, k=2, ffn=192),
    custom("mx8_shared", 161, T=70, d=128, E=16, k=4, ffn=64, n_shared=1, ffn_shared=128,
           bias="normal", bias_var=0.5),
    custom("mx8_one_token", 162, T=1, d=192, E=8, k=2, ffn=128),
    custom("mx8_stages", 163, T=64, d=1280, E=8, k=2, ffn=1024),
    custom("mx8_long_k", 164, T=24, d=4096, E=4, k=2, ffn=128),
]}


@functools.lru_cache(maxsize=None)
def case8_of(name):
    return MxCase(SMALL8[name], fmt="mxfp8")


@pytest.mark.parametrize("name", list(SMALL8))
def test_mxfp8_small(name):
    c = case8_of(name)
    x, W = c.upload()
    assert W.format == "mxfp8"
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward_mx(x, W, c.cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"{name}: max|err|/rms = {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("T", [1, 8, 32, 128, 512])
def test_mxfp8_gpt_oss_full_size(T):
    """The gpt-oss-shaped layer with MXFP8 experts: routing and y on every
    token."""
    cfg = NAMED["gpt_oss"]
    li = tables.layer_inputs(cfg, T)
    c = MxCase(cfg, T, x=li.x, fmt="mxfp8")
    x, W = c.upload()
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward_mx(x, W, cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    err = rel_err(y.cpu().numpy(), ref.y)
    print(f"gpt_oss mxfp8 T={T}: max|err|/rms = {err:.3e}")
    assert err <= TOL["bf16"], err


def _full_range_mxfp8(cfg, case):
    """Replace the MXFP8 test weights of ``case`` by codes drawn uniformly over
    all 254 non-NaN E4M3 codes (every exponent field, subnormals included;
    values 2^-9 .. 448), with each block's E8M0 scale chosen so that the
    block's rms is the dense recipe's 1/sqrt(fan_in)."""
    import oracle
    table = np.array([oracle.e4m3_value(c) for c in range(256)])

    def fill(codes, fan_in, tensor):
        c = generate.mx8_full_range_codes(cfg, codes.shape, tensor)
        blk = table[c].reshape(*c.shape[:-1], c.shape[-1] // 32, 32)
        rms = np.sqrt(np.mean(blk ** 2, axis=-1))
        sc = np.rint(127 + np.log2((1.0 / np.sqrt(fan_in)) / rms)).astype(np.int64)
        return c, np.clip(sc, 1, 254).astype(np.uint8)

    u, us, g, gs, d, ds = case.mx
    u, us = fill(u, cfg.d, 0)
    g, gs = fill(g, cfg.d, 1)
    d, ds = fill(d, cfg.ffn, 2)
    case.mx = (u, us, g, gs, d, ds)
    return np.concatenate([u.ravel(), g.ravel(), d.ravel()])


def test_mxfp8_full_code_range():
    """MXFP8 experts whose codes span the whole E4M3 range, subnormals and the
    largest finite values included.  Weights spread over 2^-9 .. 448 times a
    scale let a few products dominate, so y is held on every element to the
    h-rounding bound (twice the bf16 rounding of h, carried through the
    combine, from the oracle's fp64 h) rather than to 2e-2 * rms(y); routing
    stays exact."""
    import oracle
    cfg = custom("mx8_full_range", 165, T=200, d=512, E=16, k=4, ffn=384)
    c = MxCase(cfg, fmt="mxfp8")
    codes = _full_range_mxfp8(cfg, c)
    fields = set(((codes >> 3) & 15).tolist())
    assert fields == set(range(16)) and not np.isin(codes, [0x7F, 0xFF]).any()
    x, W = c.upload()
    ref = c.oracle()
    y, idx, w, counts = moe.moe_forward_mx(x, W, cfg.k, return_routing=True)
    torch.cuda.synchronize()
    check_routing(idx, w, counts, ref)
    yg = y.cpu().numpy().astype(np.float64)
    X = oracle.widen(c.x, "bf16")
    groups = ((e, tuple(oracle.dequant_mxfp8(*m) for m in c.expert(e))) for e in range(cfg.E))
    bound = h_rounding_bound(X, ref, groups, cfg.E, cfg.d)
    rms = float(np.sqrt(np.mean(ref.y ** 2)))
    excess = np.abs(yg - ref.y) - bound
    print(f"mxfp8 full code range: max|err|/rms = {rel_err(yg, ref.y):.3e}, "
          f"largest excess over the bound {excess.max() / rms:.2e} rms")
    assert excess.max() <= 1e-5 * rms, excess.max()


def _same_layer(x, W0, W1, k):
    y0, i0, w0, c0 = moe.moe_forward_mx(x, W0, k, return_routing=True)
    y1, i1, w1, c1 = moe.moe_forward_mx(x, W1, k, return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(w0, w1) and torch.equal(c0, c1)
    assert torch.equal(y0, y1), float((y0 - y1).abs().max())


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("name", list(SMALL))
def test_mx_line_rows_small(name, fmt):
    """MX code rows padded to whole 128-byte lines give exactly the packed
    layout's routing and y (both kernels, shared experts, partial tiles;
    rows of 32 to 2048 code bytes, on and off line boundaries)."""
    c = MxCase(SMALL[name], fmt=fmt)
    x, W0 = c.upload()
    _, W1 = c.upload(line_rows=True)
    _same_layer(x, W0, W1, c.cfg.k)


@functools.lru_cache(maxsize=None)
def _gpt_oss_case(fmt):
    cfg = NAMED["gpt_oss"]
    li = tables.layer_inputs(cfg, 128)
    return MxCase(cfg, 128, x=li.x, fmt=fmt)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_line_rows_gpt_oss(fmt):
    """The gpt-oss-shaped layer (rows of 1440 or 2880 code bytes, off line
    boundaries) with line-padded code rows at T = 1, 8 and 128 (the MXFP4
    direct-load kernel at T = 1, the LDS-staged one after): identical to the
    packed layout."""
    c = _gpt_oss_case(fmt)
    x, W0 = c.upload()
    _, W1 = c.upload(line_rows=True)
    for T in (1, 8, 128):
        _same_layer(x[:T].contiguous(), W0, W1, c.cfg.k)
    del W0, W1
    torch.cuda.empty_cache()


def test_mx_line_rows_desc_flag():
    """The flag rides in the descriptor only for padded layers."""
    c = case_of("mx_ragged")
    _, W0 = c.upload()
    _, W1 = c.upload(line_rows=True)
    assert W0.desc(8, 2).flags == 0
    assert W1.desc(8, 2).flags == moe._lib.FLAG_MX_LINE_ROWS
