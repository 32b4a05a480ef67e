"""Seeded test layers of arbitrary shape, with the routing margin enforced by
the fp64 oracle (tests may call the oracle; the product path may not)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

import oracle
from moe_inputs import generate, tables
from moe_inputs.configs import MoEConfig


def custom(name: str, cid: int, T: int, d: int, E: int, k: int, ffn: int, n_shared: int = 0,
           ffn_shared: int = 0, dtype: str = "bf16", bias: str = "none", bias_var: float = 0.0,
           margin: float = 1e-3, seed: int = 0) -> MoEConfig:
    return MoEConfig(name=name, config_id=cid, T=T, d=d, E=E, k=k, ffn=ffn, n_shared=n_shared,
                     ffn_shared=ffn_shared, dtype=dtype, bias=bias, bias_var=bias_var,
                     margin=margin, seed=seed, table=None)


def bias_of(cfg: MoEConfig) -> Optional[np.ndarray]:
    if cfg.bias == "normal":
        return generate.normal_bias(cfg)
    if cfg.bias == "none":
        return None
    return tables.router_bias(cfg)


def margin_x(cfg: MoEConfig, T: int, w_r: np.ndarray, bias, scoring: str = "softmax") -> np.ndarray:
    """First T stream rows whose top-(k+1) selection-key gaps reach cfg.margin
    (keys: the logits, or sigmoid scores plus bias for sigmoid scoring)."""
    if T == 0:
        return generate.x_stream(cfg, 0)
    n = int(T * 1.2) + 32
    while True:
        xs = generate.x_stream(cfg, n)
        if cfg.margin <= 0:
            return xs[:T]
        X, Wr = oracle.widen(xs, cfg.dtype), oracle.widen(w_r, cfg.dtype)
        if scoring == "softmax":
            K = oracle.router_logits(X, Wr, bias)
        else:
            L = oracle.router_logits(X, Wr, None)
            K = oracle.selection_keys(L, oracle.sigmoid(L), bias, scoring)
        ok = np.nonzero(oracle.topk_gaps(K, cfg.k) >= cfg.margin)[0]
        if len(ok) >= T:
            return np.ascontiguousarray(xs[ok[:T]])
        n *= 2


@dataclass(frozen=True)
class Options:
    """Router options of a case (the oracle's arguments of the same names)."""
    scoring: str = "softmax"
    renormalize: bool = True
    capacity_factor: Optional[float] = None


@dataclass
class Case:
    cfg: MoEConfig
    x: np.ndarray
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    up: np.ndarray
    gate: np.ndarray
    down: np.ndarray
    s_up: Optional[np.ndarray] = None
    s_gate: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None
    opts: Options = Options()

    def expert(self, e):
        return self.up[e], self.gate[e], self.down[e]

    def shared(self, s):
        return self.s_up[s], self.s_gate[s], self.s_down[s]

    def oracle(self, tokens=None) -> "oracle.MoEResult":
        c = self.cfg
        o = self.opts
        return oracle.moe_forward(self.x, self.w_router, self.bias, c.k, self.expert, c.E,
                                  c.dtype, self.shared if c.n_shared else None, c.n_shared,
                                  tokens, scoring=o.scoring, renormalize=o.renormalize,
                                  capacity_factor=o.capacity_factor)


def make_case(cfg: MoEConfig, T: Optional[int] = None, opts: Options = Options()) -> Case:
    """Seeded layer of `cfg` with T tokens.  Named layers with the default
    scoring read their kept rows from the stored tables; otherwise the rows
    are filtered here by the margin on the scoring's selection keys."""
    T = cfg.T if T is None else T
    w_r = generate.router_weight(cfg)
    bias = bias_of(cfg)
    if cfg.table is not None and opts.scoring == "softmax":
        li = tables.layer_inputs(cfg, T)
        x = li.x
    else:
        x = margin_x(cfg, T, w_r, bias, opts.scoring)
    up, gate, down = generate.stacked_experts(cfg)
    c = Case(cfg, x, w_r, bias, up, gate, down, opts=opts)
    if cfg.n_shared:
        c.s_up, c.s_gate, c.s_down = generate.stacked_experts(cfg, shared=True)
    return c
