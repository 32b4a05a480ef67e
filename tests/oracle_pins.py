"""Checks that tie the fp64 oracle to facts fixed by the source pages and by
mathematics, independently of the oracle's own code.  Each check raises
AssertionError on a mismatch; ``test_oracle_pins.py`` runs them and
``test_oracle_mutations.py`` plants mistakes in the oracle to show that each
check notices.

Independent means: the expected values come from the pages' printed numbers,
from closed forms, from brute force over all k-subsets / all experts, or from
library routines (torch.nn.functional, scipy.special), never from re-running
the oracle's formula.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import oracle.moe as om

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example
def worked_example_inputs():
    """The page's toy layer, built with torch's seeded init in the page's order
    (router, then each expert's two linear layers, then the tokens)."""
    g = golden("worked_example_routing.json")["model"]
    torch.manual_seed(g["seed"])
    router = torch.nn.Linear(g["d_model"], g["num_experts"], bias=False)
    experts = []
    for _ in range(g["num_experts"]):
        up = torch.nn.Linear(g["d_model"], g["d_ff"], bias=False)
        down = torch.nn.Linear(g["d_ff"], g["d_model"], bias=False)
        experts.append((up, down))
    x = torch.randn(g["tokens"], g["d_model"])
    return (x.double().numpy(), router.weight.detach().double().numpy(), experts, g)


def check_worked_example_routing():
    """Pins router logits, softmax, top-k and counts on the page's own inputs
    (P4 worked example: first token's experts, tokens per expert, experts
    touched by growing prefixes, balance loss, capacity drop)."""
    G = golden("worked_example_routing.json")
    x, wr, _, g = worked_example_inputs()
    L, P, idx, w = om.route(x, wr, None, g["k"])
    assert idx[0].tolist() == G["first_token_experts"], idx[0]
    counts = om.expert_counts(idx, g["num_experts"])
    assert counts.tolist() == G["tokens_per_expert"], counts
    for n, touched in G["experts_touched_after_tokens"].items():
        c = om.expert_counts(idx[: int(n)], g["num_experts"])
        assert int(np.sum(c > 0)) == touched, (n, c)
    f = counts / counts.sum()
    loss = g["num_experts"] * float(np.sum(f * P.mean(axis=0)))
    assert round(loss, 4) == G["balance_loss_rounded_4"], loss
    cap = math.ceil(g["tokens"] * g["k"] / g["num_experts"] * 1.25)
    assert int(np.clip(counts - cap, 0, None).sum()) == G["capacity_factor_1_25_dropped"]
    # P4 "Softmax before or after the top-k step": softmax over the kept logits
    kept = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    w2 = scipy.special.softmax(kept, axis=1)
    assert np.max(np.abs(w2 - w)) < 1e-14
    assert np.max(np.abs(w2 - w)) < G["softmax_order_max_difference_below"]


# ---------------------------------------------------------------- random layers
def rand_layer(seed, T, d, E, k, f, n_shared=0, f_sh=0, bias=True, square=False):
    rng = np.random.default_rng(seed)
    if square:
        f = d
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d)
    b = rng.standard_normal(E) * 0.7 if bias else None
    ex = [(rng.standard_normal((f, d)) / np.sqrt(d), rng.standard_normal((f, d)) / np.sqrt(d),
           rng.standard_normal((d, f)) / np.sqrt(f)) for _ in range(E)]
    sh = [(rng.standard_normal((f_sh, d)) / np.sqrt(d), rng.standard_normal((f_sh, d)) / np.sqrt(d),
           rng.standard_normal((d, f_sh)) / np.sqrt(f_sh)) for _ in range(n_shared)]
    return x, wr, b, ex, sh


def torch_ffn(xrow, wu, wg, wd):
    """SwiGLU expert with library routines (torch fp64 CPU)."""
    X = torch.from_numpy(np.atleast_2d(xrow))
    h = F.silu(F.linear(X, torch.from_numpy(wg))) * F.linear(X, torch.from_numpy(wu))
    return F.linear(h, torch.from_numpy(wd)).numpy()


def brute_force_y(x, wr, b, ex, sh, k):
    """Dense evaluation (page "Mixture of Experts Explained: Routers, Active Parameters and VRAM",
    "Why MoE models can feel fast anyway": the loop matched a slow version
    that runs every expert with zero weight for the unpicked ones): every token through every
    expert, gated by a length-E vector that is zero off the top-k.  The top-k
    set is the k-subset with the largest logit sum, over all subsets; the
    weights are library softmax probabilities renormalised over that set."""
    T, d = x.shape
    E = wr.shape[0]
    L = x @ wr.T + (0 if b is None else b)
    P = scipy.special.softmax(L, axis=1)
    y = np.zeros((T, d))
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(L[t, list(s)]))
        gate = np.zeros(E)
        gate[list(best)] = P[t, list(best)] / P[t, list(best)].sum()
        for e in range(E):
            y[t] += gate[e] * torch_ffn(x[t], *ex[e])[0]
        for s in sh:
            y[t] += torch_ffn(x[t], *s)[0]
    return y


def run_oracle_f64(x, wr, b, ex, sh, k):
    """Call the oracle on float64 arrays (store them as 'f32' is not exact, so
    pass fp64 straight through widen's f32 branch, which is astype(float64))."""
    return om.moe_forward(x, wr, b, k, lambda e: ex[e], wr.shape[0], "f32",
                          (lambda s: sh[s]) if sh else None, len(sh))


def check_brute_force(seed=1, T=24, d=16, E=6, k=3, f=20, n_shared=1, square=False):
    x, wr, b, ex, sh = rand_layer(seed, T, d, E, k, f, n_shared, f, square=square)
    r = run_oracle_f64(x, wr, b, ex, sh, k)
    yb = brute_force_y(x, wr, b, ex, sh, k)
    err = np.max(np.abs(r.y - yb)) / np.sqrt(np.mean(yb ** 2))
    assert err < 1e-12, err


def check_topk_bruteforce(seed=2, T=200, E=7, k=3):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E))
    idx = om.select_topk(L, k)
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(L[t, list(s)]))
        assert set(idx[t].tolist()) == set(best)
        vals = L[t, idx[t]]
        assert np.all(vals[:-1] > vals[1:])


def check_tie_break():
    """Exact ties go to the lower expert index (the layer's stated tie rule)."""
    L = np.array([[0.5, 0.7, 0.7, 0.1],
                  [0.7, 0.5, 0.7, 0.7],
                  [0.0, 0.0, 0.0, 0.0],
                  [-1.0, 2.0, -1.0, 2.0]])
    assert om.select_topk(L, 2).tolist() == [[1, 2], [0, 2], [0, 1], [1, 3]]
    assert om.select_topk(L, 1).tolist() == [[1], [0], [0], [1]]
    assert om.select_topk(L, 4)[2].tolist() == [0, 1, 2, 3]


def check_softmax_library(seed=3):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((50, 33)) * 4
    assert np.max(np.abs(om.softmax(L) - scipy.special.softmax(L, axis=1))) < 1e-15


def check_invariants(seed=4, T=300, E=16, k=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, 24))
    wr = rng.standard_normal((E, 24))
    L, P, idx, w = om.route(x, wr, rng.standard_normal(E), k)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-14
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
        assert np.all(np.diff(L[t, idx[t]]) < 0)
    counts = om.expert_counts(idx, E)
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    order = om.dispatch_order(idx, E)
    assert np.array_equal(order, np.argsort(idx.ravel(), kind="stable"))
    # k = 1: renormalised weight is exactly one (P4 "Why top-1 routing cannot renormalise")
    _, _, _, w1 = om.route(x, wr, None, 1)
    assert np.all(w1 == 1.0)


def check_uniform_gates():
    """All-zero router: every logit ties, so with k = E each weight is 1/E and
    y is the mean of all experts; with k < E it is the mean of experts 0..k-1."""
    rng = np.random.default_rng(5)
    T, d, E, f = 6, 12, 5, 10
    x, _, _, ex, _ = rand_layer(5, T, d, E, E, f, bias=False)
    wr = np.zeros((E, d))
    for k in (E, 2):
        r = run_oracle_f64(x, wr, None, ex, [], k)
        ref = np.mean([torch_ffn(x, *ex[e]) for e in range(k)], axis=0)
        assert np.max(np.abs(r.y - ref)) < 1e-13, k
        assert np.all(r.idx == np.arange(k)[None, :])
    del rng


def check_single_expert_library():
    """E = 1, k = 1 reduces to one dense SwiGLU FFN (torch library)."""
    x, wr, _, ex, _ = rand_layer(6, 9, 16, 1, 1, 24, bias=False)
    r = run_oracle_f64(x, wr, None, ex, [], 1)
    assert np.max(np.abs(r.y - torch_ffn(x, *ex[0]))) < 1e-13


def check_silu():
    z = np.linspace(-30, 30, 601)
    assert np.max(np.abs(om.silu(z) - F.silu(torch.from_numpy(z)).numpy())) < 1e-14
    # z*s(z) - (-z)*s(-z) = z, since s(z) + s(-z) = 1
    assert np.max(np.abs(om.silu(z) - om.silu(-z) - z)) < 1e-12
    assert om.silu(np.array([0.0]))[0] == 0.0


def check_widen():
    vals = torch.randn(1000, dtype=torch.float32) * 3
    b = vals.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(om.widen(bits, "bf16"), b.double().numpy())


def check_occupancy_table():
    G = golden("occupancy_table.json")
    for key, row in G["share_touched_percent_1dp"].items():
        parts = key.split("_")
        k, E = int(parts[1][1:]), int(parts[2][1:])
        for B, pct in zip(G["batches"], row):
            assert round(100 * om.share_touched(k, E, B), 1) == pct, (key, B)
    M = G["mixtral_weights_read"]
    expert_B = (M["total_params_B"] - M["active_params_B"]) / (1 - M["k"] / M["E"])
    other_B = M["total_params_B"] - expert_B
    for B, pct, wread in zip(M["batches"], M["experts_touched_percent"], M["weights_read_B"]):
        s = om.share_touched(M["k"], M["E"], B)
        assert round(100 * s, 1) == pct
        assert abs(other_B + s * expert_B - wread) <= 0.1 + 1e-9, (B, other_B + s * expert_B)


def check_occupancy_monte_carlo(trials=3000, seed=7):
    """Routing with iid logits is uniform over k-subsets, so the mean touched
    share matches the closed form (page "Mixture of experts: how MoE works
    and what it costs", "How batching changes the mixture of experts math": a
    Monte Carlo run agreed within 0.05 percentage points)."""
    rng = np.random.default_rng(seed)
    for k, E, B in ((2, 8, 4), (8, 256, 16), (4, 128, 8)):
        shares = np.empty(trials)
        for i in range(trials):
            idx = om.select_topk(rng.standard_normal((B, E)), k)
            shares[i] = np.sum(om.expert_counts(idx, E) > 0) / E
        se = shares.std() / np.sqrt(trials)
        assert abs(shares.mean() - om.share_touched(k, E, B)) < 4 * se + 1e-12, (k, E, B)


# ---------------------------------------------------------------- router variants
def check_sigmoid_library():
    z = np.linspace(-60, 60, 1201)
    assert np.max(np.abs(om.sigmoid(z) - scipy.special.expit(z))) < 1e-15
    assert om.sigmoid(np.array([0.0]))[0] == 0.5


def check_sigmoid_bias_selection_only():
    """Closed forms of sigmoid scoring with a selection-only bias: the bias
    decides which experts are kept, the weights use the scores alone."""
    x = np.eye(3)
    wr = np.array([[3.0, 0.0, 0.0], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]])  # L = [3, 0, 0] for token 0
    b = np.array([0.0, 0.5, 0.25])
    L, S, idx, w = om.route(x[:1], wr, b, 1, scoring="sigmoid")
    assert L[0].tolist() == [3.0, 0.0, 0.0]                  # no bias in the logits
    assert idx[0].tolist() == [1]                            # 0.5 + 0.5 > 1/(1+e^-3) > 0.5 + 0.25
    assert w[0].tolist() == [1.0]
    _, _, idx2, w2 = om.route(x[:1], wr, b, 2, scoring="sigmoid")
    s3 = 1.0 / (1.0 + math.exp(-3.0))
    assert idx2[0].tolist() == [1, 0]
    assert np.allclose(w2[0], [0.5 / (0.5 + s3), s3 / (0.5 + s3)], rtol=0, atol=1e-15)
    _, _, idx3, w3 = om.route(x[:1], wr, b, 2, scoring="sigmoid", renormalize=False)
    assert idx3[0].tolist() == [1, 0] and np.allclose(w3[0], [0.5, s3], rtol=0, atol=1e-15)
    # without a bias the choice is the logit order (sigmoid is increasing)
    _, _, idx4, _ = om.route(x[:1], wr, None, 3, scoring="sigmoid")
    assert idx4[0].tolist() == [0, 1, 2]


def check_sigmoid_routing_bruteforce(seed=21, T=150, d=10, E=7, k=3):
    """Sigmoid routing against brute force over all k-subsets: the kept set
    maximises the sum of (expit(logit) + bias), listed by decreasing key; the
    weights are library expit scores over that set, renormalised or raw."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d) * 3
    b = rng.standard_normal(E) * 0.3
    L, S, idx, w = om.route(x, wr, b, k, scoring="sigmoid")
    _, _, idx_r, w_r = om.route(x, wr, b, k, scoring="sigmoid", renormalize=False)
    Lref = x @ wr.T
    sref = scipy.special.expit(Lref)
    assert np.max(np.abs(L - Lref)) < 1e-12
    for t in range(T):
        key = sref[t] + b
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(key[list(c)]))
        order = sorted(best, key=lambda e: -key[e])
        assert idx[t].tolist() == order and idx_r[t].tolist() == order
        kept = sref[t, order]
        assert np.max(np.abs(w[t] - kept / kept.sum())) < 1e-14
        assert np.max(np.abs(w_r[t] - kept)) < 1e-15


def check_raw_softmax_weights(seed=22, T=80, d=12, E=6):
    """Raw weights under softmax scoring are the library softmax probabilities
    of the kept experts; with k = E they sum to one; renormalised top-1
    weights are exactly one (P4 "Why top-1 routing cannot renormalise")."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    b = rng.standard_normal(E)
    Pref = scipy.special.softmax(x @ wr.T + b, axis=1)
    for k in (1, 3, E):
        _, _, idx, w = om.route(x, wr, b, k, renormalize=False)
        assert np.max(np.abs(w - np.take_along_axis(Pref, idx.astype(np.int64), axis=1))) < 1e-15
        if k == E:
            assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-14
        _, _, _, wn = om.route(x, wr, b, k)
        if k == 1:
            assert np.all(wn == 1.0)


def check_capacity_closed_forms():
    """The capacity formula of page "Mixture of Experts Explained: Routers, Active Parameters and VRAM",
    "Noise and the second expert": ceil(tokens * k / experts * factor).  On the page's
    printed tokens-per-expert list (512 tokens, top-2, 8 experts) factor 1.0
    gives 128 and drops (135-128)+(147-128)+(133-128) = 31 slots; factors 1.25
    and 2.0 drop none (the page: an even router drops nothing at 1.25)."""
    G = golden("worked_example_routing.json")
    counts = np.array(G["tokens_per_expert"])
    assert om.expert_capacity(512, 2, 8, 1.0) == 128
    assert om.expert_capacity(512, 2, 8, 1.25) == 160
    assert om.expert_capacity(512, 2, 8, 2.0) == 256
    assert om.expert_capacity(10, 2, 3, 1.0) == 7       # 6.67 rounds up
    assert om.expert_capacity(3, 1, 4, 0.5) == 1        # 0.375 rounds up
    # pairs in an order that has the printed counts: expert of pair p
    flat = np.repeat(np.arange(8), counts)
    rng = np.random.default_rng(23)
    rng.shuffle(flat)
    idx = flat.reshape(512, 2)
    for factor, dropped in ((1.0, 7 + 19 + 5), (1.25, G["capacity_factor_1_25_dropped"]), (2.0, 0)):
        keep = om.capacity_keep(idx, 8, om.expert_capacity(512, 2, 8, factor))
        assert int((~keep).sum()) == dropped, factor


def _keep_by_sort(idx, E, cap):
    """Independent form of the capacity rule: stable-sort the pairs by expert;
    a pair is kept when its position inside its expert's run is below cap."""
    flat = np.asarray(idx).ravel()
    order = np.argsort(flat, kind="stable")
    starts = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))[:-1]])
    pos = np.empty(len(flat), dtype=np.int64)
    pos[order] = np.arange(len(flat)) - starts[flat[order]]
    return (pos < cap).reshape(np.asarray(idx).shape)


def check_capacity_bruteforce(seed=24):
    """Capacity keep-mask against the sort-based form, per-expert kept counts
    min(count, capacity), and every dropped pair after every kept pair of its
    expert; then y against a dense evaluation with the dropped gates zeroed."""
    rng = np.random.default_rng(seed)
    for T, E, k, factor in ((40, 5, 2, 1.0), (64, 8, 3, 0.6), (7, 3, 3, 2.0), (50, 6, 1, 0.25)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if k > 1 else \
            rng.integers(0, 2, size=(T, 1))  # skewed: experts 0 and 1 only
        cap = om.expert_capacity(T, k, E, factor)
        keep = om.capacity_keep(idx, E, cap)
        assert np.array_equal(keep, _keep_by_sort(idx, E, cap)), (T, E, k, factor)
        counts = np.bincount(idx.ravel(), minlength=E)
        kept = np.bincount(idx.ravel()[keep.ravel()], minlength=E)
        assert np.array_equal(kept, np.minimum(counts, cap))
        for e in range(E):
            ks = keep.ravel()[idx.ravel() == e]
            assert np.all(np.diff(ks.astype(int)) <= 0)
    # the whole layer: skewed router so some pairs drop
    T, d, E, k, f = 30, 10, 4, 2, 12
    x, wr, b, ex, sh = rand_layer(25, T, d, E, k, f, n_shared=1, f_sh=8)
    b = np.array([2.0, 1.0, 0.0, -1.0])
    factor = 0.75
    r = om.moe_forward(x, wr, b, k, lambda e: ex[e], E, "f32", lambda s: sh[s], 1,
                       capacity_factor=factor)
    L = x @ wr.T + b
    P = scipy.special.softmax(L, axis=1)
    sets = [sorted(max(itertools.combinations(range(E), k), key=lambda c: sum(L[t, list(c)])),
                   key=lambda e: -L[t, e]) for t in range(T)]
    idx = np.array(sets)
    keep = _keep_by_sort(idx, E, math.ceil(T * k / E * factor))
    assert (~keep).sum() > 0
    assert np.array_equal(r.keep, keep)
    y = np.zeros((T, d))
    for t in range(T):
        g = P[t, idx[t]] / P[t, idx[t]].sum()
        for j in range(k):
            if keep[t, j]:
                y[t] += g[j] * torch_ffn(x[t], *ex[idx[t, j]])[0]
        y[t] += torch_ffn(x[t], *sh[0])[0]
    assert np.max(np.abs(r.y - y)) / np.sqrt(np.mean(y ** 2)) < 1e-12


def check_sigmoid_layer_bruteforce(seed=26, T=20, d=12, E=5, k=2, f=16):
    """The whole layer with sigmoid scoring against a dense evaluation."""
    x, wr, b, ex, sh = rand_layer(seed, T, d, E, k, f)
    r = om.moe_forward(x, wr, b, k, lambda e: ex[e], E, "f32", scoring="sigmoid")
    s = scipy.special.expit(x @ wr.T)
    y = np.zeros((T, d))
    for t in range(T):
        key = s[t] + b
        best = list(max(itertools.combinations(range(E), k), key=lambda c: sum(key[list(c)])))
        gate = np.zeros(E)
        gate[best] = s[t, best] / s[t, best].sum()
        for e in range(E):
            y[t] += gate[e] * torch_ffn(x[t], *ex[e])[0]
    assert np.max(np.abs(r.y - y)) / np.sqrt(np.mean(y ** 2)) < 1e-12


# ---------------------------------------------------------------- MXFP4 expert weights
def check_e2m1_table():
    """The E2M1 element values of the OCP MX format: codes 0..7 are
    0, 0.5, 1, 1.5, 2, 3, 4, 6 and codes 8..15 their negatives."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert om.e2m1_value(c) == mags[c]
        assert om.e2m1_value(c + 8) == -mags[c]
        assert math.copysign(1.0, om.e2m1_value(c + 8)) == -1.0


def check_e8m0_library():
    """E8M0 scale bytes against torch's float8_e8m0fnu conversion."""
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).float().double().numpy()
    got = np.array([om.e8m0_value(int(v)) for v in range(256)])
    assert np.array_equal(got[:255], ref[:255]) and np.isnan(got[255]) and np.isnan(ref[255])


def _dequant_loop(codes, scales):
    """Element by element: element k of row n is nibble k % 2 (low first) of
    byte k // 2, times the scale of block k // 32."""
    N, half = codes.shape
    out = np.empty((N, 2 * half))
    for n in range(N):
        for k in range(2 * half):
            code = (int(codes[n, k // 2]) >> (4 * (k % 2))) & 0xF
            out[n, k] = om.e2m1_value(code) * 2.0 ** (int(scales[n, k // 32]) - 127)
    return out


def check_mxfp4_dequant(seed=27):
    """Dequantisation against the element-by-element form, and a hand-made
    row: byte 0x21 holds 0.5 (low nibble) then 1.0; the second block's scale
    byte 129 multiplies it by 4."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(5, 48), dtype=np.uint8)
    scales = rng.integers(110, 140, size=(5, 3), dtype=np.uint8)
    assert np.array_equal(om.dequant_mxfp4(codes, scales), _dequant_loop(codes, scales))
    row = np.full((1, 32), 0x21, dtype=np.uint8)
    d = om.dequant_mxfp4(row, np.array([[127, 129]], dtype=np.uint8))[0]
    assert d[:4].tolist() == [0.5, 1.0, 0.5, 1.0] and d[32:34].tolist() == [2.0, 4.0]


def check_mxfp4_layer_bruteforce(seed=28, T=12, d=64, E=4, k=2, f=32):
    """The layer with MXFP4 experts equals a dense evaluation on the
    element-by-element dequantised weights."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d)
    mx = [tuple((rng.integers(0, 256, size=(r, c // 2), dtype=np.uint8),
                 rng.integers(120, 125, size=(r, c // 32), dtype=np.uint8))
                for r, c in ((f, d), (f, d), (d, f))) for _ in range(E)]
    r = om.moe_forward(x, wr, None, k, lambda e: mx[e], E, "f32", expert_dtype="mxfp4")
    dense = [tuple(_dequant_loop(*m) for m in mx[e]) for e in range(E)]
    P = scipy.special.softmax(x @ wr.T, axis=1)
    y = np.zeros((T, d))
    for t in range(T):
        best = sorted(max(itertools.combinations(range(E), k),
                          key=lambda c: sum((x @ wr.T)[t, list(c)])))
        g = P[t, best] / P[t, best].sum()
        for j, e in enumerate(best):
            y[t] += g[j] * torch_ffn(x[t], *dense[e])[0]
    assert np.max(np.abs(r.y - y)) / np.sqrt(np.mean(y ** 2)) < 1e-12


# ---------------------------------------------------------------- MXFP8 expert weights
def check_e4m3_library():
    """All 256 E4M3 codes against torch's float8_e4m3fn conversion (NaN at
    0x7F and 0xFF, no infinity)."""
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([om.e4m3_value(v) for v in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])


def check_e4m3_closed_forms():
    """Codes whose values the format fixes: 0x38 = 1 (exponent field 7 =
    bias), 0xB8 = -1, 0x7E = 1.75 * 2^8 = 448 (the largest), 0x08 = 2^-6
    (the smallest normal), 0x01 = 2^-9 (the smallest subnormal), 0x00 = 0."""
    for code, v in [(0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0x08, 2.0 ** -6),
                    (0x01, 2.0 ** -9), (0x00, 0.0), (0x3C, 1.5), (0x40, 2.0)]:
        assert om.e4m3_value(code) == v, (hex(code), om.e4m3_value(code))
    assert math.isnan(om.e4m3_value(0x7F)) and math.isnan(om.e4m3_value(0xFF))


def check_mxfp8_dequant(seed=29):
    """Dequantisation against torch's E4M3 values element by element, each
    times the E8M0 scale of its 32-element block, and a hand-made row."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(4, 96), dtype=np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scales = rng.integers(110, 140, size=(4, 3), dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ref = ref * 2.0 ** (scales.astype(np.int64)[:, np.arange(96) // 32] - 127)
    assert np.array_equal(om.dequant_mxfp8(codes, scales), ref)
    row = np.full((1, 64), 0x38, dtype=np.uint8)
    d = om.dequant_mxfp8(row, np.array([[127, 130]], dtype=np.uint8))[0]
    assert d[:32].tolist() == [1.0] * 32 and d[32:].tolist() == [8.0] * 32


def check_mxfp8_layer_bruteforce(seed=30, T=10, d=64, E=3, k=2, f=32):
    """The layer with MXFP8 experts equals a dense evaluation on torch's
    E4M3 values times the block scales."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d)

    def draw(r, c):
        codes = rng.integers(0, 256, size=(r, c), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x30
        return codes, rng.integers(118, 124, size=(r, c // 32), dtype=np.uint8)

    mx = [tuple(draw(r, c) for r, c in ((f, d), (f, d), (d, f))) for _ in range(E)]
    r = om.moe_forward(x, wr, None, k, lambda e: mx[e], E, "f32", expert_dtype="mxfp8")

    def dense(codes, scales):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
        return v * 2.0 ** (scales.astype(np.int64)[:, np.arange(codes.shape[1]) // 32] - 127)

    P = scipy.special.softmax(x @ wr.T, axis=1)
    y = np.zeros((T, d))
    for t in range(T):
        best = sorted(max(itertools.combinations(range(E), k),
                          key=lambda c: sum((x @ wr.T)[t, list(c)])))
        g = P[t, best] / P[t, best].sum()
        for j, e in enumerate(best):
            y[t] += g[j] * torch_ffn(x[t], *(dense(*m) for m in mx[e]))[0]
    assert np.max(np.abs(r.y - y)) / np.sqrt(np.mean(y ** 2)) < 1e-12


# ---------------------------------------------------------------- routing margin
def _gap_pairs(row, k):
    """Smallest |L_a - L_b| over pairs whose first member is one of the k kept
    experts (found as the k-subset with the largest sum, over all subsets) and
    whose second is any other expert.  Pairs with both members outside the
    kept set do not bound how far the kept list can move."""
    E = len(row)
    if E < 2:
        return math.inf
    best = max(itertools.combinations(range(E), k), key=lambda c: sum(row[list(c)]))
    return min(abs(row[a] - row[b]) for a in best for b in range(E) if b != a)


def _ordered_topk(row, k):
    """The kept experts in descending score order, ties to the lower index,
    by Python's sort on (-score, index)."""
    return sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]


def check_topk_gaps_hand_rows():
    """Rows with a known smallest gap, placed inside the kept list, between the
    last kept and the first dropped expert, or only among dropped experts
    (which must not count), each in shuffled column order; k = E; E = 1."""
    rows = [  # (row, k, gap)
        ([3.0, 2.9999, 1.0, 0.0], 2, 1e-4),          # inside the kept list
        ([3.0, 2.0, 1.9999, 0.0], 2, 1e-4),          # between ranks k and k+1
        ([3.0, 2.0, 1.0, 0.9999], 2, 1.0),           # only between dropped ranks
        ([3.0, 2.0, 1.0, 0.5, 0.49999], 3, 0.5),     # ranks k+1 and k+2 do not count
        ([5.0, 4.0, 3.5, -1.0, -1.0], 3, 0.5),       # exact tie among dropped experts
        ([0.25, 1.5, 1.0], 3, 0.5),                  # k = E: every consecutive gap
        ([0.25, 1.5, 1.0], 2, 0.5),                  # E = k + 1
        ([2.0, 2.0, 1.0], 1, 0.0),                   # tie at the top
        ([7.0, -3.0], 1, 10.0),
    ]
    rng = np.random.default_rng(31)
    for row, k, gap in rows:
        for _ in range(4):
            perm = rng.permutation(len(row))
            got = om.topk_gaps(np.array(row)[perm][None, :], k)[0]
            assert abs(got - gap) < 1e-12, (row, k, gap, got)
    assert om.topk_gaps(np.array([[1.3]]), 1)[0] == math.inf


def check_topk_gaps_pairs(seed=32):
    """Against the pair brute force on random rows (some with repeated values),
    for every k from 1 to E."""
    rng = np.random.default_rng(seed)
    for E in (2, 3, 5, 8):
        L = np.round(rng.standard_normal((60, E)) * 3, 1)  # coarse grid: ties happen
        for k in range(1, E + 1):
            got = om.topk_gaps(L, k)
            want = np.array([_gap_pairs(L[t], k) for t in range(L.shape[0])])
            assert np.allclose(got, want, rtol=0, atol=1e-12), (E, k)


def check_topk_gaps_meaning(seed=33):
    """What the margin promises: a row whose gap is g keeps the same ordered
    top k under any perturbation smaller than g/2 in every entry, and a
    perturbation of g/2 (plus a little) aimed at the pair that realises the
    gap changes it."""
    rng = np.random.default_rng(seed)
    for E, k in ((6, 2), (8, 3), (4, 4), (5, 1)):
        L = rng.standard_normal((40, E))
        g = om.topk_gaps(L, k)
        for t in range(L.shape[0]):
            base = _ordered_topk(L[t], k)
            for _ in range(20):
                d = rng.uniform(-1, 1, E) * g[t] / 2 * (1 - 1e-9)
                assert _ordered_topk(L[t] + d, k) == base, (E, k, t)
            # the realising pair: a kept expert a and any other b at distance g
            pairs = [(a, b) for a in base for b in range(E)
                     if b != a and abs(L[t, a] - L[t, b]) <= g[t] * (1 + 1e-12)]
            assert pairs, (E, k, t)
            a, b = pairs[0]
            hi, lo = (a, b) if L[t, a] > L[t, b] else (b, a)
            d = np.zeros(E)
            step = g[t] / 2 * (1 + 1e-6) + 1e-12
            d[hi] -= step
            d[lo] += step
            assert _ordered_topk(L[t] + d, k) != base, (E, k, t)


# ---------------------------------------------------------------- Zipf target
def zipf_shares(E, s):
    """Zipf(s) over ranks 1..E: p_r = r^-s / sum_q q^-s, summed term by term."""
    w = [1.0 / r ** s for r in range(1, E + 1)]
    tot = math.fsum(w)
    return [v / tot for v in w]


def check_zipf_targets(E=32, s=1.1):
    """The mid-size layer's target load shares are Zipf(1.1) over the 32
    experts, expert r-1 at rank r: both the stored table (6 decimals) and the
    table script's target function."""
    from oracle import make_input_tables as mit
    want = zipf_shares(E, s)
    for target, atol in ((golden_table("midsize_zipf")["target_shares"], 5e-7),
                         (list(mit.zipf_target(E, s)), 1e-15)):
        assert len(target) == E
        assert max(abs(a - b) for a, b in zip(target, want)) <= atol, (target[:3], want[:3])
    assert len(target) == E
    assert max(abs(a - b) for a, b in zip(target, want)) <= atol, (target[:3], want[:3])
    # spot values: the hottest expert takes 28.4%, the coldest 0.63%
    assert round(100 * want[0], 1) == 28.4 and round(100 * want[-1], 2) == 0.63


def golden_table(name):
    tab = os.path.join(os.path.dirname(GOLDEN), os.pardir, "moe_inputs", "tables", name + ".json")
    with open(tab) as f:
        return json.load(f)


ALL = [check_worked_example_routing, check_brute_force, check_topk_bruteforce, check_tie_break,
       check_softmax_library, check_invariants, check_uniform_gates,
       check_single_expert_library, check_silu, check_widen, check_occupancy_table,
       check_occupancy_monte_carlo, check_sigmoid_library, check_sigmoid_bias_selection_only,
       check_sigmoid_routing_bruteforce, check_raw_softmax_weights, check_capacity_closed_forms,
       check_capacity_bruteforce, check_sigmoid_layer_bruteforce, check_e2m1_table,
       check_e8m0_library, check_mxfp4_dequant, check_mxfp4_layer_bruteforce,
       check_e4m3_library, check_e4m3_closed_forms, check_mxfp8_dequant,
       check_mxfp8_layer_bruteforce, check_topk_gaps_hand_rows, check_topk_gaps_pairs,
       check_topk_gaps_meaning, check_zipf_targets]
