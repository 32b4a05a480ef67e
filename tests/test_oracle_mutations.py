"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin.

Each case swaps one oracle function for a plausible wrong version and checks
that at least the named pin fails."""
import numpy as np
import pytest

import oracle.moe as om
import oracle_pins as P


def _ties_to_high(L, k):
    T, E = L.shape
    e_ix = np.broadcast_to(-np.arange(E), (T, E))
    return np.lexsort((e_ix, -L), axis=-1)[:, :k].astype(np.int32)


def _no_renorm(Pm, idx):
    return np.take_along_axis(Pm, idx.astype(np.int64), axis=-1)


def _swapped_swiglu(X, wu, wg, wd):
    return (om.silu(X @ wu.T) * (X @ wg.T)) @ wd.T


def _transposed_down(X, wu, wg, wd):
    return (om.silu(X @ wg.T) * (X @ wu.T)) @ wd


def _no_bias(x, w, bias=None):
    return x @ w.T


def _sign_silu(z):
    return z / (1.0 + np.exp(z))


def _ascending(L, k):
    T, E = L.shape
    e_ix = np.broadcast_to(np.arange(E), (T, E))
    return np.lexsort((e_ix, L), axis=-1)[:, :k].astype(np.int32)


def _counts_off_by_one(idx, E):
    flat = np.asarray(idx).ravel()
    return np.array([int(np.sum(flat == e + 1)) for e in range(E)], dtype=np.int32)


def _unstable_order(idx, E):
    return np.argsort(np.asarray(idx).ravel(), kind="quicksort")[::-1].astype(np.int64)


def _sigmoid_of_biased_logit(L, Pm, bias, scoring):
    if scoring == "sigmoid" and bias is not None:
        return om.sigmoid(L + np.asarray(bias)[None, :])
    return L if scoring == "softmax" else Pm


def _sign_sigmoid(z):
    return 1.0 / (1.0 + np.exp(z))


def _keep_last(idx, E, capacity):
    idx = np.asarray(idx)
    flat = idx.ravel()[::-1]
    taken = np.zeros(E, dtype=np.int64)
    keep = np.zeros(flat.shape, dtype=bool)
    for p, e in enumerate(flat.tolist()):
        keep[p] = taken[e] < capacity
        taken[e] += 1
    return keep[::-1].reshape(idx.shape)


def _capacity_floor(T, k, E, factor):
    return int(T * k / E * factor)


def _capacity_per_token(T, k, E, factor):
    return int(np.ceil(T / E * factor))


def _e2m1_bias2(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 2) * (1.0 + 0.5 * m)
    return -mag if s else mag


def _e8m0_bias128(byte):
    return 2.0 ** (int(byte) - 128)


def _dequant_high_nibble_first(codes, scales):
    swapped = ((np.asarray(codes) & 0xF) << 4) | (np.asarray(codes) >> 4)
    return _REAL_DEQUANT(swapped.astype(np.uint8), scales)


def _dequant_block16(codes, scales):
    codes = np.asarray(codes)
    N, half = codes.shape
    el = _REAL_DEQUANT(codes, np.full((N, 2 * half // 32), 127, np.uint8))
    nb = np.asarray(scales).shape[1]
    sc = 2.0 ** (np.asarray(scales, np.int64)[:, np.arange(2 * half // 16) % nb] - 127)
    return (el.reshape(N, -1, 16) * sc[:, :, None]).reshape(N, -1)


_REAL_DEQUANT = om.dequant_mxfp4


def _e4m3_bias8(code):
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -7 * (m / 8.0) if e == 0 else 2.0 ** (e - 8) * (1.0 + m / 8.0)
    return -mag if s else mag


def _e4m3_no_subnormals(code):
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 0.0 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def _dequant8_block16(codes, scales):
    codes = np.asarray(codes)
    N, K = codes.shape
    table = np.array([om.e4m3_value(c) for c in range(256)])
    nb = np.asarray(scales).shape[1]
    sc = 2.0 ** (np.asarray(scales, np.int64)[:, (np.arange(K) // 16) % nb] - 127)
    return table[codes] * sc

def _gaps_last_only(L, k):
    s = -np.sort(-L, axis=-1)[:, :min(k + 1, L.shape[1])]
    if s.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    return s[:, -2] - s[:, -1]


def _gaps_k_values(L, k):
    s = -np.sort(-L, axis=-1)[:, :k]
    if s.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    return np.min(s[:, :-1] - s[:, 1:], axis=-1)


def _gaps_k_plus_2(L, k):
    s = -np.sort(-L, axis=-1)[:, :k + 2]
    if s.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    return np.min(s[:, :-1] - s[:, 1:], axis=-1)


def _gaps_ascending(L, k):
    s = np.sort(L, axis=-1)[:, :min(k + 1, L.shape[1])]
    if s.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    return np.min(np.abs(s[:, :-1] - s[:, 1:]), axis=-1)


def _gaps_unsorted(L, k):
    s = L[:, :min(k + 1, L.shape[1])]
    if s.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    return np.min(np.abs(s[:, :-1] - s[:, 1:]), axis=-1)


def _zipf_wrong_exponent(E, s):
    r = np.arange(1, E + 1, dtype=np.float64)
    t = r ** (-1.0)
    return t / t.sum()


def _zipf_from_zero(E, s):
    r = np.arange(0, E, dtype=np.float64) + 2.0
    t = r ** (-s)
    return t / t.sum()


MUTANTS = [
    ("topk_gaps", _gaps_last_only, P.check_topk_gaps_hand_rows),
    ("topk_gaps", _gaps_last_only, P.check_topk_gaps_pairs),
    ("topk_gaps", _gaps_k_values, P.check_topk_gaps_hand_rows),
    ("topk_gaps", _gaps_k_values, P.check_topk_gaps_meaning),
    ("topk_gaps", _gaps_k_plus_2, P.check_topk_gaps_hand_rows),
    ("topk_gaps", _gaps_k_plus_2, P.check_topk_gaps_pairs),
    ("topk_gaps", _gaps_ascending, P.check_topk_gaps_hand_rows),
    ("topk_gaps", _gaps_unsorted, P.check_topk_gaps_pairs),
    ("e2m1_value", _e2m1_bias2, P.check_e2m1_table),
    ("e8m0_value", _e8m0_bias128, P.check_e8m0_library),
    ("dequant_mxfp4", _dequant_high_nibble_first, P.check_mxfp4_dequant),
    ("dequant_mxfp4", _dequant_block16, P.check_mxfp4_dequant),
    ("dequant_mxfp4", _dequant_high_nibble_first, P.check_mxfp4_layer_bruteforce),
    ("e4m3_value", _e4m3_bias8, P.check_e4m3_library),
    ("e4m3_value", _e4m3_bias8, P.check_e4m3_closed_forms),
    ("e4m3_value", _e4m3_no_subnormals, P.check_e4m3_library),
    ("dequant_mxfp8", _dequant8_block16, P.check_mxfp8_dequant),
    ("dequant_mxfp8", _dequant8_block16, P.check_mxfp8_layer_bruteforce),
    ("selection_keys", _sigmoid_of_biased_logit, P.check_sigmoid_bias_selection_only),
    ("sigmoid", _sign_sigmoid, P.check_sigmoid_library),
    ("sigmoid", _sign_sigmoid, P.check_sigmoid_routing_bruteforce),
    ("capacity_keep", _keep_last, P.check_capacity_bruteforce),
    ("expert_capacity", _capacity_floor, P.check_capacity_closed_forms),
    ("expert_capacity", _capacity_per_token, P.check_capacity_closed_forms),
    ("kept_scores", lambda Pm, idx: om.renormalise(Pm, idx), P.check_raw_softmax_weights),
    ("select_topk", _ties_to_high, P.check_tie_break),
    ("select_topk", _ascending, P.check_worked_example_routing),
    ("renormalise", _no_renorm, P.check_invariants),
    ("renormalise", _no_renorm, P.check_brute_force),
    ("swiglu_expert", _swapped_swiglu, P.check_single_expert_library),
    ("swiglu_expert", _transposed_down,
     lambda: P.check_brute_force(seed=11, T=16, d=12, E=5, k=2, n_shared=0, square=True)),
    ("router_logits", _no_bias, P.check_brute_force),
    ("silu", _sign_silu, P.check_silu),
    ("expert_counts", _counts_off_by_one, P.check_worked_example_routing),
    ("dispatch_order", _unstable_order, P.check_invariants),
]


@pytest.mark.parametrize("name,bad,check", MUTANTS,
                         ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, bad, check):
    monkeypatch.setattr(om, name, bad)
    with pytest.raises(AssertionError):
        check()


ZIPF_MUTANTS = [_zipf_wrong_exponent, _zipf_from_zero]


@pytest.mark.parametrize("bad", ZIPF_MUTANTS, ids=lambda f: f.__name__)
def test_zipf_mutant_is_caught(monkeypatch, bad):
    from oracle import make_input_tables as mit
    monkeypatch.setattr(mit, "zipf_target", bad)
    with pytest.raises(AssertionError):
        P.check_zipf_targets()


def test_dropped_shared_expert_is_caught(monkeypatch):
    real = om.moe_forward

    def no_shared(x, wr, b, k, efn, E, dtype, shared_fn=None, n_shared=0, tokens=None):
        return real(x, wr, b, k, efn, E, dtype, None, 0, tokens)
    monkeypatch.setattr(om, "moe_forward", no_shared)
    with pytest.raises(AssertionError):
        P.check_brute_force()
