"""Stored per-layer tables: which token-stream rows are kept, and the Zipf bias.

A table is JSON written by ``oracle/make_input_tables.py`` (which computes
router logits with the fp64 oracle).  This module only reads it and picks the
listed rows; it computes nothing about the layer.

Fields: ``rows_needed`` (how many kept rows the table covers), ``stream_rows``
(how many stream rows that takes), ``rejected`` (stream row indices dropped
because their top-(k+1) logit gaps were below the margin) and, for the Zipf
recipe, ``bias_f32_hex`` (the calibrated float32 bias as hex bit patterns).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from . import generate
from .configs import MoEConfig

TABLE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tables")


def table_path(name: str) -> str:
    return os.path.join(TABLE_DIR, name + ".json")


def load_table(name: str) -> Dict:
    with open(table_path(name)) as f:
        return json.load(f)


def bias_from_hex(hexes: List[str]) -> np.ndarray:
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def bias_to_hex(b: np.ndarray) -> List[str]:
    return ["%08x" % int(v) for v in np.asarray(b, np.float32).view(np.uint32)]


def router_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    """The float32 router logit bias of a layer, or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return generate.normal_bias(cfg)
    if cfg.bias == "zipf":
        if cfg.table is None:
            raise ValueError("zipf bias needs a stored table")
        return bias_from_hex(load_table(cfg.table)["bias_f32_hex"])
    raise ValueError(cfg.bias)


def kept_rows(cfg: MoEConfig, T: int) -> np.ndarray:
    """Stream indices of the first T kept rows, from the stored table."""
    tab = load_table(cfg.table)
    if T > tab["rows_needed"]:
        raise ValueError(f"table {cfg.table} covers {tab['rows_needed']} rows, asked {T}")
    rej = set(tab["rejected"])
    out = [i for i in range(tab["stream_rows"]) if i not in rej]
    return np.asarray(out[:T], dtype=np.int64)


@dataclass
class LayerInputs:
    cfg: MoEConfig
    x: np.ndarray                    # [T, d] stored type
    w_router: np.ndarray             # [E, d]
    bias: Optional[np.ndarray]       # [E] float32 or None
    stream_rows: np.ndarray          # stream index of each x row


def layer_inputs(cfg: MoEConfig, T: Optional[int] = None) -> LayerInputs:
    """x, router weight and bias of a named layer at T tokens, using the stored
    row table.  Expert weights are drawn separately (they are large)."""
    T = cfg.T if T is None else T
    rows = kept_rows(cfg, T)
    n = int(rows[-1]) + 1 if len(rows) else 0
    xs = generate.x_stream(cfg, n)
    return LayerInputs(cfg, np.ascontiguousarray(xs[rows]), generate.router_weight(cfg),
                       router_bias(cfg), rows)
