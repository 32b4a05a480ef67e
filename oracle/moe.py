"""The plain fp64 definition of one sparse top-k MoE layer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, cited by page title and section:

* P1 "Mixture of Experts (MoE): routing, expert parallelism, and memory",
  sections "How does MoE routing work" and "Shared experts".
* P2 "Mixture of Experts: why a model with 671 billion parameters uses only
  37", sections "Where MoE changes the Transformer", "The router: how a token
  chooses experts" (pseudo-PyTorch layer) and "Shared expert and fine-grained
  experts".
* P3 "Mixture of experts: how MoE works and what it costs", sections "What
  mixture of experts costs in compute" and "How batching changes the mixture
  of experts math" (occupancy closed form).
* P4 "Mixture of Experts Explained: Routers, Active Parameters and VRAM", the
  five numbered routing steps (Score, Normalise, Keep the top k, Renormalise,
  Run and combine), the gated three-matrix feed-forward remark, the worked
  example and "Softmax before or after the top-k step".

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):

* the gated expert is SwiGLU: h = SiLU(x W_gate^T) * (x W_up^T), out = h W_down^T,
  with SiLU(z) = z / (1 + exp(-z)) and no biases;
* selection keeps the k largest logits in descending order; an exact tie goes
  to the lower expert index; selection is done on logits (softmax is monotone,
  so the chosen set and order are the same as on probabilities);
* the kept probabilities are renormalised to sum to one (P4 step 4);
* a per-expert bias, when present, is added to the logits before the softmax;
* shared experts are added with coefficient one; no residual term is added.

Router variants (not the default layer; selected by arguments):

* sigmoid scoring (P2 "How many experts to pick and how to score them: top-k,
  softmax, sigmoid"): each expert's score is sigmoid(logit) on its own; the
  per-expert balancing bias (P2 "The problem learned routing brings: load
  balancing"; P3 "Why load balancing is the hard part of MoE": the bias moves
  routing but not the gate values) is added to the scores for selection only;
  the weights are the kept scores, renormalised over the kept set;
* raw weights (P4 "Why top-1 routing cannot renormalise"): the kept scores
  (softmax probabilities over all experts, or sigmoid scores) are used as they
  are, without renormalising;
* expert capacity (P2 "Capacity factor: when tokens don't fit"; P4, the
  capacity passage after the balance-loss example in "Noise and the second
  expert"): capacity = ceil(T*k/E * factor), the P4 form over routing slots
  (P2 writes tokens per batch over experts; with top-k each token fills k
  slots); each expert takes the first `capacity` (token, slot) pairs that
  chose it in pair order t*k+j, and a pair beyond that skips the expert, so
  its term is missing from y (the token would pass on through the residual
  connection, which this layer does not add).

Low-bit expert weights (P2 "What to do about it in practice": experts take 4
bits well, gpt-oss ships them in MXFP4; P3 "What mixture of experts costs in
memory": MXFP4 expert weights; P4 "Why MoE models can feel fast anyway": 4
bits per weight).  The pages name the format without defining it; the
definition used is the OCP Microscaling (MX) format MXFP4: blocks of 32
consecutive elements along K share one E8M0 scale 2^(S-127); each element is
FP4 E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is
subnormal: 0 or 0.5).  Two elements per byte, element 2i in the low nibble.
The layer computes with the dequantized weights exactly as with stored
bf16/f32 weights.  For the 8-bit expert weights the pages mention (P3 "What
mixture of experts costs in memory": DeepSeek-V3's weights are mostly 8-bit)
the same MX blocking is used with FP8 E4M3 elements (MXFP8: bias 7, no
infinity, 0x7F/0xFF NaN), one element per byte.

Parity status: every function here is pinned by a CPU test against the pages'
printed worked example, closed forms, brute force or a library routine, except
the Zipf bias calibration in ``make_input_tables.py``, whose outcome is an
input recipe and is parity unpinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence, Tuple

import numpy as np


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.  'bf16' storage is the upper 16 bits
    of an IEEE float32, so shifting the pattern left by 16 gives the float32
    with the same value."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: (-1)^s * (e == 0 ? m/2 : 2^(e-1) * (1 + m/2))."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale byte: 2^(byte - 127); 255 is NaN."""
    return float("nan") if byte == 255 else 2.0 ** (int(byte) - 127)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix -> float64.  codes [N, K/2] uint8 (element 2i in the low
    nibble of byte i), scales [N, K/32] uint8 -> [N, K] = element * scale of
    its 32-element block along K."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, half = codes.shape
    K = 2 * half
    if scales.shape != (N, K // 32) or K % 32:
        raise ValueError("MXFP4 shapes")
    table = np.array([e2m1_value(c) for c in range(16)])
    el = np.empty((N, K), dtype=np.float64)
    el[:, 0::2] = table[codes & 0xF]
    el[:, 1::2] = table[codes >> 4]
    sc = np.array([e8m0_value(b) for b in range(256)])[scales]
    return (el.reshape(N, K // 32, 32) * sc[:, :, None]).reshape(N, K)


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code (OCP FP8, the element of MXFP8): sign,
    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (2^-6 * m/8); 0x7F and 0xFF (exponent and mantissa all ones) are NaN and
    there is no infinity, so the largest magnitude is 1.75 * 2^8 = 448."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 (E4M3 elements) matrix -> float64.  codes [N, K] uint8, scales
    [N, K/32] uint8 -> [N, K] = element * scale of its 32-element block."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, K = codes.shape
    if scales.shape != (N, K // 32) or K % 32:
        raise ValueError("MXFP8 shapes")
    table = np.array([e4m3_value(c) for c in range(256)])
    sc = np.array([e8m0_value(b) for b in range(256)])[scales]
    return (table[codes].reshape(N, K // 32, 32) * sc[:, :, None]).reshape(N, K)


def widen_weight(w, dtype: str) -> np.ndarray:
    """A stored weight matrix -> float64: a bf16/f32 array, or for 'mxfp4' /
    'mxfp8' a (codes, scales) pair."""
    if dtype == "mxfp4":
        return dequant_mxfp4(*w)
    if dtype == "mxfp8":
        return dequant_mxfp8(*w)
    return widen(w, dtype)


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """P1 "How does MoE routing work" step 1, P2 "The router", P4 step
    "Score": one score per expert = token hidden state times the E x d router
    matrix (a bias-free linear layer).  The optional per-expert bias is added
    here.  x [T,d] f64, w_router [E,d] f64 -> logits [T,E] f64."""
    L = x @ w_router.T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def softmax(L: np.ndarray) -> np.ndarray:
    """P4 step "Normalise": probabilities over all E experts, summing to 1."""
    m = L.max(axis=-1, keepdims=True)
    e = np.exp(L - m)
    return e / e.sum(axis=-1, keepdims=True)


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """P4 step "Keep the top k": the k largest scores of each token, in
    descending order; an exact tie goes to the lower expert index.  Returns
    int32 [T,k]."""
    T, E = L.shape
    e_ix = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((e_ix, -L), axis=-1)  # primary: -L ascending; then e
    return order[:, :k].astype(np.int32)


def renormalise(P: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """P4 step "Renormalise": divide the k kept probabilities by their sum."""
    kept = np.take_along_axis(P, idx.astype(np.int64), axis=-1)
    return kept / kept.sum(axis=-1, keepdims=True)


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Independent per-expert score in (0, 1): 1 / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def kept_scores(P: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """The scores of the k kept experts, as they are (no renormalising)."""
    return np.take_along_axis(P, idx.astype(np.int64), axis=-1)


def selection_keys(L: np.ndarray, P: np.ndarray, bias: Optional[np.ndarray],
                   scoring: str) -> np.ndarray:
    """What the top-k step ranks.  softmax: the logits (bias already in L).
    sigmoid: the scores plus the per-expert bias, which only steers the
    choice."""
    if scoring == "softmax":
        return L
    if scoring == "sigmoid":
        return P if bias is None else P + np.asarray(bias, np.float64)[None, :]
    raise ValueError(scoring)


def route(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray], k: int,
          scoring: str = "softmax", renormalize: bool = True):
    """Router: logits L, per-expert scores P (softmax probabilities, or
    sigmoid scores), top-k indices and weights.  Softmax scoring adds the bias
    to the logits; sigmoid scoring leaves it out of L and P and adds it to the
    selection keys only.  Weights are the kept scores, renormalised unless
    ``renormalize`` is false."""
    if scoring == "softmax":
        L = router_logits(x, w_router, bias)
        P = softmax(L)
    elif scoring == "sigmoid":
        L = router_logits(x, w_router, None)
        P = sigmoid(L)
    else:
        raise ValueError(scoring)
    idx = select_topk(selection_keys(L, P, bias, scoring), k)
    w = renormalise(P, idx) if renormalize else kept_scores(P, idx)
    return L, P, idx, w


def expert_capacity(T: int, k: int, E: int, factor: float) -> int:
    """Most (token, slot) pairs one expert takes: ceil(T*k/E * factor),
    evaluated in that order in IEEE double (page "Mixture of Experts Explained: Routers, Active Parameters and VRAM",
    "Noise and the second expert": its capacity formula)."""
    return math.ceil(T * k / E * factor)


def capacity_keep(idx: np.ndarray, E: int, capacity: int) -> np.ndarray:
    """bool [T,k]: pair (t, j) is kept when fewer than `capacity` pairs with a
    smaller pair id t'*k+j' chose the same expert."""
    idx = np.asarray(idx)
    flat = idx.ravel()
    taken = np.zeros(E, dtype=np.int64)
    keep = np.zeros(flat.shape, dtype=bool)
    for p, e in enumerate(flat.tolist()):
        keep[p] = taken[e] < capacity
        taken[e] += 1
    return keep.reshape(idx.shape)


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """Tokens per expert: how many (token, slot) pairs chose each expert (the
    per-expert count printed in the P4 worked example).  int32 [E]."""
    flat = np.asarray(idx).ravel()
    return np.array([int(np.sum(flat == e)) for e in range(E)], dtype=np.int32)


def dispatch_order(idx: np.ndarray, E: int) -> np.ndarray:
    """Grouping of (token, slot) pairs by expert (P2 "The router" pseudo-layer
    loops experts and gathers the tokens that chose each; P3 "What mixture of
    experts costs in compute": tokens are grouped by expert before each
    multiply).  Returns the flat pair ids t*k+j, expert 0's first, each
    expert's pairs in increasing pair id."""
    flat = np.asarray(idx).ravel()
    parts = [np.nonzero(flat == e)[0] for e in range(E)]
    return (np.concatenate(parts) if parts else np.zeros(0, np.int64)).astype(np.int64)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(X: np.ndarray, w_up: np.ndarray, w_gate: np.ndarray,
                  w_down: np.ndarray) -> np.ndarray:
    """One gated expert FFN (page "Mixture of Experts Explained: Routers, Active Parameters and VRAM",
    the active-parameter arithmetic: a gated block with three matrices; page
    "Mixture of Experts: why a model with 671 billion parameters uses only
    37", "Where MoE changes the Transformer": two linear layers with an
    activation between them): SiLU(X W_gate^T) * (X W_up^T), then times W_down^T.
    X [n,d]; w_up, w_gate [f,d]; w_down [d,f] -> [n,d]."""
    U = X @ w_up.T
    G = X @ w_gate.T
    return (silu(G) * U) @ w_down.T


def topk_gaps(L: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between consecutive logits among the k+1 largest of each
    token (the k largest when k equals E).  A token whose gap is at least a
    margin m has a top-k set and order that any logit error below m/2 cannot
    change."""
    T, E = L.shape
    s = -np.sort(-L, axis=-1)[:, :min(k + 1, E)]
    if s.shape[1] < 2:
        return np.full(T, np.inf)
    return np.min(s[:, :-1] - s[:, 1:], axis=-1)


def share_touched(k: int, E: int, B: int) -> float:
    """P3 "How batching changes the mixture of experts math": expected share
    of the E experts used by at least one of B tokens when each token picks k
    distinct experts uniformly at random: 1 - (1 - k/E)^B."""
    return 1.0 - (1.0 - k / E) ** B


@dataclass
class MoEResult:
    y: np.ndarray          # [n_tokens, d] float64 (rows of `tokens`)
    idx: np.ndarray        # [T, k] int32
    w: np.ndarray          # [T, k] float64
    counts: np.ndarray     # [E] int32
    logits: np.ndarray     # [T, E] float64
    probs: np.ndarray      # [T, E] float64
    tokens: np.ndarray     # token ids y covers
    keep: np.ndarray       # [T, k] bool: pair taken by its expert (all True without capacity)


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def moe_forward(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray], k: int,
                expert_fn: ExpertFn, E: int, dtype: str,
                shared_fn: Optional[ExpertFn] = None, n_shared: int = 0,
                tokens: Optional[Sequence[int]] = None, scoring: str = "softmax",
                renormalize: bool = True,
                capacity_factor: Optional[float] = None,
                expert_dtype: Optional[str] = None) -> MoEResult:
    """The whole layer (P4 step "Run and combine"; P1 "Shared experts"):

        y[t] = sum_{j<k} w[t,j] * FFN_{idx[t,j]}(x[t]) + sum_s FFN_shared_s(x[t])

    summed in slot order j = 0..k-1, then the shared experts.  Only the
    experts that some token chose are evaluated, each on just its tokens.

    x and w_router are stored arrays (``dtype`` 'f32' or 'bf16' bit patterns);
    expert_fn(e) / shared_fn(s) return the stored (W_up, W_gate, W_down) of an
    expert.  Routing is computed for all T tokens; y only for ``tokens``
    (default: all), so large layers can be checked on a sample.
    ``scoring`` / ``renormalize`` pick the router variant (see ``route``);
    with a ``capacity_factor`` the pairs beyond an expert's capacity (which
    depends on every token's routing) add nothing to y.  ``expert_dtype``
    ('mxfp4') stores the expert weights (routed and shared) in another
    format than x and the router (default: ``dtype``).
    """
    edt = dtype if expert_dtype is None else expert_dtype
    X = widen(x, dtype)
    L, P, idx, w = route(X, widen(w_router, dtype), bias, k, scoring, renormalize)
    T = X.shape[0]
    counts = expert_counts(idx, E)
    if capacity_factor is None:
        keep = np.ones(idx.shape, dtype=bool)
    else:
        keep = capacity_keep(idx, E, expert_capacity(T, k, E, capacity_factor))
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    # per (sampled token, slot) expert output, then a slot-ordered sum
    slot_out = np.zeros((len(tok), k, X.shape[1]))
    order = dispatch_order(idx[tok], E)
    sub_idx = idx[tok].ravel()
    start = 0
    for e in range(E):
        n_e = int(np.sum(sub_idx == e))
        if n_e == 0:
            continue
        pairs = order[start:start + n_e]
        start += n_e
        rows = pairs // k
        wu, wg, wd = (widen_weight(a, edt) for a in expert_fn(e))
        out = swiglu_expert(X[tok[rows]], wu, wg, wd)
        slot_out[rows, pairs % k] = out
    y = np.zeros((len(tok), X.shape[1]))
    wt = w[tok]
    kt = keep[tok]
    for j in range(k):
        y += np.where(kt[:, j:j + 1], wt[:, j:j + 1] * slot_out[:, j], 0.0)
    for s in range(n_shared):
        su, sg, sd = (widen_weight(a, edt) for a in shared_fn(s))
        y += swiglu_expert(X[tok], su, sg, sd)
    return MoEResult(y, idx, w, counts, L, P, tok, keep)
