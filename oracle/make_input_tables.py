"""Write the stored row/bias tables of the named synthetic layers.

TEST INFRASTRUCTURE (input preparation): calls only the fp64 oracle and the
seeded generator; nothing here is read back from a GPU.

For each named layer:

1. Zipf layers: calibrate a float32 per-expert logit bias so that the share of
   (token, slot) pairs routed to expert r-1 approaches r^-s / sum_q q^-s.  The
   update is a damped fixed point on the log shares,
   b <- b + 0.5 * ln(target / measured), 60 rounds from b = ln(target), with
   routing computed by the oracle on the first T raw stream rows.  (Parity
   unpinned: this only shapes the inputs; the routing it produces is pinned
   exactly against the oracle.)
2. Margin: walk the token stream and keep a row only if every gap between
   consecutive logits among its top k+1 is at least ``cfg.margin`` (fp64
   logits of the stored, already-rounded inputs).  Record the rejected rows.

Run:  python -m oracle.make_input_tables [name ...]
"""
from __future__ import annotations

import json
import sys
import time

import numpy as np

from moe_inputs import NAMED, generate, tables
from moe_inputs.configs import MoEConfig

from . import moe


def zipf_target(E: int, s: float) -> np.ndarray:
    """Zipf(s) load shares over ranks r = 1..E: r^-s / sum_q q^-s."""
    r = np.arange(1, E + 1, dtype=np.float64)
    target = r ** (-s)
    return target / target.sum()


def calibrate_zipf(cfg: MoEConfig, x_raw: np.ndarray, w_r: np.ndarray, rounds: int = 60):
    E, k = cfg.E, cfg.k
    target = zipf_target(E, cfg.zipf_s)
    L0 = moe.router_logits(moe.widen(x_raw, cfg.dtype), moe.widen(w_r, cfg.dtype), None)
    b = np.log(target)
    for _ in range(rounds):
        bf = b.astype(np.float32)
        idx = moe.select_topk(L0 + bf.astype(np.float64)[None, :], k)
        meas = np.maximum(moe.expert_counts(idx, E), 0.5) / (x_raw.shape[0] * k)
        b = bf.astype(np.float64) + 0.5 * np.log(target / meas)
    return b.astype(np.float32), target


def kept_rows(cfg: MoEConfig, w_r: np.ndarray, bias, need: int):
    n = int(need * 1.15) + 64
    while True:
        xs = generate.x_stream(cfg, n)
        L = moe.router_logits(moe.widen(xs, cfg.dtype), moe.widen(w_r, cfg.dtype), bias)
        gaps = moe.topk_gaps(L, cfg.k)
        ok = gaps >= cfg.margin
        if ok.sum() >= need:
            last = int(np.nonzero(ok)[0][need - 1])
            stream_rows = last + 1
            rejected = [int(i) for i in np.nonzero(~ok[:stream_rows])[0]]
            return stream_rows, rejected, float(gaps[:stream_rows][ok[:stream_rows]].min())
        n *= 2


def make(cfg: MoEConfig) -> dict:
    t0 = time.time()
    w_r = generate.router_weight(cfg)
    out = {"config": cfg.name, "margin": cfg.margin, "rows_needed": cfg.t_max}
    bias = None
    if cfg.bias == "zipf":
        x_raw = generate.x_stream(cfg, cfg.T)
        b, target = calibrate_zipf(cfg, x_raw, w_r)
        out["bias_f32_hex"] = tables.bias_to_hex(b)
        out["target_shares"] = [round(float(v), 6) for v in target]
        bias = b
    elif cfg.bias == "normal":
        bias = generate.normal_bias(cfg)
    stream_rows, rejected, min_gap = kept_rows(cfg, w_r, bias, cfg.t_max)
    out.update(stream_rows=stream_rows, rejected=rejected, min_kept_gap=min_gap,
               redraw_rate=round(len(rejected) / stream_rows, 5))
    if cfg.bias == "zipf":
        xs = generate.x_stream(cfg, stream_rows)
        keep = np.setdiff1d(np.arange(stream_rows), np.asarray(rejected, np.int64))[:cfg.T]
        L = moe.router_logits(moe.widen(xs[keep], cfg.dtype), moe.widen(w_r, cfg.dtype), bias)
        counts = moe.expert_counts(moe.select_topk(L, cfg.k), cfg.E)
        out["achieved_shares"] = [round(float(c) / (cfg.T * cfg.k), 6) for c in counts]
    out["seconds"] = round(time.time() - t0, 2)
    return out


def main(names):
    for name in names or list(NAMED):
        cfg = NAMED[name]
        tab = make(cfg)
        with open(tables.table_path(cfg.table), "w") as f:
            json.dump(tab, f, indent=1)
        print(name, "stream_rows", tab["stream_rows"], "rejected", len(tab["rejected"]),
              "min_gap %.2e" % tab["min_kept_gap"], "%.1fs" % tab["seconds"])


if __name__ == "__main__":
    main(sys.argv[1:])
