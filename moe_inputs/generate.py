"""Seeded synthetic inputs for the sparse-MoE layer.

This module is shared by the fp64 oracle and by the GPU path, and it holds no
arithmetic of the layer itself: it only draws random numbers, scales them to
the requested standard deviation, rounds them to the storage type and returns
the stored bit patterns.  Row selection for the routing margin and the Zipf
bias calibration are computed elsewhere and stored as small tables under
``tables/`` (see ``tables.py``).

Recipe (all draws are numpy PCG64 streams keyed by
``SeedSequence([seed, config_id, tensor_id, expert_id])``):

* values are drawn as float32 standard normals, multiplied by the float32
  standard deviation (one float32 rounding), and for bf16 layers rounded
  once more to bfloat16 with round-to-nearest-even;
* x ~ N(0, 1), one stream of rows [T_stream, d];
* router weight [E, d] ~ N(0, 1/d);
* per routed expert e: W_up, W_gate [ffn, d] ~ N(0, 1/d), W_down [d, ffn]
  ~ N(0, 1/ffn); shared experts likewise with ffn_shared;
* router bias: 'normal' draws float64 N(0, 1) times sqrt(bias_var), stored as
  float32; 'zipf' is read from the stored table;
* MXFP4 expert weights (layers that store experts in that format): each
  matrix draws its packed E2M1 code bytes uniformly (every code equally
  likely) and one E8M0 scale byte per 32 elements along K, the byte
  round(127 + log2(std / 2.9261)) plus a uniform draw from {-1, 0, 1};
  2.9261 is the rms of the 16 equally likely E2M1 values, so the
  weights' rms is within a factor of two of the dense recipe's std.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Dict, Iterator, List, Optional, Sequence, Tuple

import numpy as np

from .configs import MoEConfig

# stream ids
X, W_ROUTER, W_UP, W_GATE, W_DOWN, WS_UP, WS_GATE, WS_DOWN, BIAS = range(9)
MX_UP, MX_GATE, MX_DOWN = range(9, 12)
MX8_UP, MX8_GATE, MX8_DOWN = range(12, 15)
MX8_FULL = 15
# rms of the E2M1 values when all 16 codes are equally likely: the values are
# 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, sqrt(68.5 / 8)
_E2M1_RMS = 2.9261
# MXFP8 test codes: any sign and mantissa, exponent field 4..9 (magnitudes
# 2^-3 .. 7.5, a spread like that of E2M1's 0.5 .. 6; codes over the whole
# E4M3 range would span 2^-9 .. 448 and let a few weights dominate); rms of
# those 96 equally likely values
_E4M3_EXP_LO, _E4M3_EXP_HI = 4, 9
_E4M3_RMS = 2.7635


def _rng(cfg: MoEConfig, tensor_id: int, expert_id: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, cfg.config_id, tensor_id, expert_id])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _draw(cfg: MoEConfig, tensor_id: int, expert_id: int, shape: Tuple[int, ...],
          std: float) -> np.ndarray:
    rng = _rng(cfg, tensor_id, expert_id)
    z = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    z = z.reshape(shape)
    if cfg.dtype == "f32":
        return z
    return f32_to_bf16_bits(z)


def x_stream(cfg: MoEConfig, n_rows: int) -> np.ndarray:
    """The first ``n_rows`` rows of the token stream, stored type, [n_rows, d].
    Row i does not depend on n_rows."""
    return _draw(cfg, X, 0, (n_rows, cfg.d), 1.0)


def router_weight(cfg: MoEConfig) -> np.ndarray:
    return _draw(cfg, W_ROUTER, 0, (cfg.E, cfg.d), 1.0 / np.sqrt(cfg.d))


def normal_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert logit bias for the 'normal' recipe, float32 [E]."""
    z = _rng(cfg, BIAS, 0).standard_normal(cfg.E)
    return (z * np.sqrt(cfg.bias_var)).astype(np.float32)


def expert_weights(cfg: MoEConfig, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(W_up [ffn,d], W_gate [ffn,d], W_down [d,ffn]) of routed expert e."""
    sd_in, sd_mid = 1.0 / np.sqrt(cfg.d), 1.0 / np.sqrt(cfg.ffn)
    return (_draw(cfg, W_UP, e, (cfg.ffn, cfg.d), sd_in),
            _draw(cfg, W_GATE, e, (cfg.ffn, cfg.d), sd_in),
            _draw(cfg, W_DOWN, e, (cfg.d, cfg.ffn), sd_mid))


def shared_weights(cfg: MoEConfig, s: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(W_up [ffn_s,d], W_gate [ffn_s,d], W_down [d,ffn_s]) of shared expert s."""
    sd_in, sd_mid = 1.0 / np.sqrt(cfg.d), 1.0 / np.sqrt(cfg.ffn_shared)
    return (_draw(cfg, WS_UP, s, (cfg.ffn_shared, cfg.d), sd_in),
            _draw(cfg, WS_GATE, s, (cfg.ffn_shared, cfg.d), sd_in),
            _draw(cfg, WS_DOWN, s, (cfg.d, cfg.ffn_shared), sd_mid))


def _workers(n: Optional[int]) -> int:
    if n:
        return n
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        c = os.cpu_count() or 1
    return max(1, min(16, c))


def iter_experts(cfg: MoEConfig, experts: Sequence[int], shared: bool = False,
                 workers: Optional[int] = None) -> Iterator[Tuple[int, Tuple[np.ndarray, ...]]]:
    """Yield (e, weights) for the given expert ids, in order, generating up to
    ``workers`` experts concurrently (numpy releases the GIL while drawing)."""
    fn = shared_weights if shared else expert_weights
    experts = list(experts)
    w = _workers(workers)
    with _cf.ThreadPoolExecutor(w) as ex:
        pending: Dict[int, _cf.Future] = {}
        nxt = 0
        for i, e in enumerate(experts):
            while nxt < len(experts) and nxt < i + 2 * w:
                pending[nxt] = ex.submit(fn, cfg, experts[nxt])
                nxt += 1
            yield e, pending.pop(i).result()


def stacked_experts(cfg: MoEConfig, shared: bool = False,
                    workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """All routed (or shared) expert weights stacked on a leading expert axis."""
    n = cfg.n_shared if shared else cfg.E
    f = cfg.ffn_shared if shared else cfg.ffn
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    up = np.empty((n, f, cfg.d), dt)
    gate = np.empty((n, f, cfg.d), dt)
    down = np.empty((n, cfg.d, f), dt)
    for e, (u, g, dn) in iter_experts(cfg, range(n), shared, workers):
        up[e], gate[e], down[e] = u, g, dn
    return up, gate, down



def _mx_draw(cfg: MoEConfig, tensor_id: int, expert_id: int, rows: int, cols: int,
             std: float) -> Tuple[np.ndarray, np.ndarray]:
    """(codes [rows, cols/2] uint8, scales [rows, cols/32] uint8) of one MXFP4
    matrix whose values have an rms within a factor of two of ``std``."""
    rng = _rng(cfg, tensor_id, expert_id)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    base = int(round(127 + np.log2(std / _E2M1_RMS)))
    scales = (base + rng.integers(-1, 2, size=(rows, cols // 32))).astype(np.uint8)
    return codes, scales


def mxfp4_expert_weights(cfg: MoEConfig, e: int, shared: bool = False):
    """((up codes, up scales), (gate codes, gate scales), (down codes, down
    scales)) of routed expert e (or shared expert e) stored as MXFP4."""
    f = cfg.ffn_shared if shared else cfg.ffn
    sd_in, sd_mid = 1.0 / np.sqrt(cfg.d), 1.0 / np.sqrt(f)
    ids = (MX_UP, MX_GATE, MX_DOWN)
    sid = 1000 + e if shared else e
    return (_mx_draw(cfg, ids[0], sid, f, cfg.d, sd_in),
            _mx_draw(cfg, ids[1], sid, f, cfg.d, sd_in),
            _mx_draw(cfg, ids[2], sid, cfg.d, f, sd_mid))


def stacked_mxfp4(cfg: MoEConfig, shared: bool = False):
    """All routed (or shared) MXFP4 experts stacked: (up, up_scale, gate,
    gate_scale, down, down_scale) uint8 arrays."""
    n = cfg.n_shared if shared else cfg.E
    f = cfg.ffn_shared if shared else cfg.ffn
    up = np.empty((n, f, cfg.d // 2), np.uint8)
    up_s = np.empty((n, f, cfg.d // 32), np.uint8)
    gate = np.empty_like(up)
    gate_s = np.empty_like(up_s)
    down = np.empty((n, cfg.d, f // 2), np.uint8)
    down_s = np.empty((n, cfg.d, f // 32), np.uint8)
    for e in range(n):
        (up[e], up_s[e]), (gate[e], gate_s[e]), (down[e], down_s[e]) = \
            mxfp4_expert_weights(cfg, e, shared)
    return up, up_s, gate, gate_s, down, down_s


def _mx8_draw(cfg: MoEConfig, tensor_id: int, expert_id: int, rows: int, cols: int,
              std: float) -> Tuple[np.ndarray, np.ndarray]:
    """(codes [rows, cols] uint8, scales [rows, cols/32] uint8) of one MXFP8
    (E4M3) matrix whose values have an rms within a factor of two of
    ``std`` (no NaN code can be drawn)."""
    rng = _rng(cfg, tensor_id, expert_id)
    sign = rng.integers(0, 2, size=(rows, cols), dtype=np.uint8)
    expo = rng.integers(_E4M3_EXP_LO, _E4M3_EXP_HI + 1, size=(rows, cols), dtype=np.uint8)
    mant = rng.integers(0, 8, size=(rows, cols), dtype=np.uint8)
    codes = (sign << 7) | (expo << 3) | mant
    base = int(round(127 + np.log2(std / _E4M3_RMS)))
    scales = (base + rng.integers(-1, 2, size=(rows, cols // 32))).astype(np.uint8)
    return codes.astype(np.uint8), scales


def mx8_full_range_codes(cfg: MoEConfig, shape: Tuple[int, ...], tensor: int) -> np.ndarray:
    """E4M3 code bytes drawn uniformly over the 254 codes that are not NaN
    (0x7F and 0xFF excluded), every exponent field included; ``tensor``
    (0, 1, 2 for up, gate, down) keys the stream."""
    rng = _rng(cfg, MX8_FULL, tensor)
    v = rng.integers(0, 254, size=shape, dtype=np.int64)
    v = v + (v >= 0x7F)          # skip 0x7F
    return v.astype(np.uint8)    # 254 -> 0xFF is never drawn: top value is 0xFE


def mxfp8_expert_weights(cfg: MoEConfig, e: int, shared: bool = False):
    """((up codes, up scales), (gate codes, gate scales), (down codes, down
    scales)) of routed expert e (or shared expert e) stored as MXFP8."""
    f = cfg.ffn_shared if shared else cfg.ffn
    sd_in, sd_mid = 1.0 / np.sqrt(cfg.d), 1.0 / np.sqrt(f)
    sid = 1000 + e if shared else e
    return (_mx8_draw(cfg, MX8_UP, sid, f, cfg.d, sd_in),
            _mx8_draw(cfg, MX8_GATE, sid, f, cfg.d, sd_in),
            _mx8_draw(cfg, MX8_DOWN, sid, cfg.d, f, sd_mid))


def stacked_mxfp8(cfg: MoEConfig, shared: bool = False):
    """All routed (or shared) MXFP8 experts stacked: (up, up_scale, gate,
    gate_scale, down, down_scale) uint8 arrays."""
    n = cfg.n_shared if shared else cfg.E
    f = cfg.ffn_shared if shared else cfg.ffn
    up = np.empty((n, f, cfg.d), np.uint8)
    up_s = np.empty((n, f, cfg.d // 32), np.uint8)
    gate = np.empty_like(up)
    gate_s = np.empty_like(up_s)
    down = np.empty((n, cfg.d, f), np.uint8)
    down_s = np.empty((n, cfg.d, f // 32), np.uint8)
    for e in range(n):
        (up[e], up_s[e]), (gate[e], gate_s[e]), (down[e], down_s[e]) = \
            mxfp8_expert_weights(cfg, e, shared)
    return up, up_s, gate, gate_s, down, down_s
