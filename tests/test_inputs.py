"""The seeded generator and the stored row/bias tables (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins as P
from moe_inputs import NAMED, generate, tables
from moe_inputs.configs import MoEConfig


def test_bf16_rounding_matches_torch():
    v = (torch.randn(200_000) * 5).float()
    v[:4] = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0])  # exact ties
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(generate.f32_to_bf16_bits(v.numpy()), ref)


def test_stream_prefix_and_determinism():
    cfg = NAMED["gpt_oss"]
    a = generate.x_stream(cfg, 7)
    b = generate.x_stream(cfg, 19)
    assert np.array_equal(a, b[:7])
    assert np.array_equal(generate.router_weight(cfg), generate.router_weight(cfg))
    u1 = generate.expert_weights(cfg, 3)[0]
    u2 = generate.expert_weights(cfg, 4)[0]
    assert not np.array_equal(u1, u2)


def test_draw_scales():
    cfg = NAMED["tiny_f32"]
    up, gate, down = generate.expert_weights(cfg, 0)
    assert up.dtype == np.float32 and up.shape == (cfg.ffn, cfg.d)
    assert abs(up.std() * np.sqrt(cfg.d) - 1) < 0.02
    assert abs(down.std() * np.sqrt(cfg.ffn) - 1) < 0.02
    x = generate.x_stream(cfg, 256)
    assert abs(x.std() - 1) < 0.02


def test_normal_bias_variance():
    cfg = MoEConfig("t", 99, 1, 8, 20000, 2, 8, bias="normal", bias_var=0.5)
    b = generate.normal_bias(cfg)
    assert b.dtype == np.float32 and abs(b.var() - 0.5) < 0.03


@pytest.mark.parametrize("name", list(NAMED))
def test_tables_reproduce(name):
    """The stored kept-row lists are what the oracle's margin rule gives, and
    the assembled inputs meet the margin."""
    cfg = NAMED[name]
    tab = tables.load_table(cfg.table)
    li = tables.layer_inputs(cfg, cfg.t_max)
    assert li.x.shape == (cfg.t_max, cfg.d)
    L = oracle.router_logits(oracle.widen(li.x, cfg.dtype), oracle.widen(li.w_router, cfg.dtype),
                             li.bias)
    assert np.min(oracle.topk_gaps(L, cfg.k)) >= cfg.margin
    xs = generate.x_stream(cfg, tab["stream_rows"])
    Ls = oracle.router_logits(oracle.widen(xs, cfg.dtype), oracle.widen(li.w_router, cfg.dtype),
                              li.bias)
    bad = np.nonzero(oracle.topk_gaps(Ls, cfg.k) < cfg.margin)[0].tolist()
    assert bad == tab["rejected"]


def test_nested_token_counts():
    cfg = NAMED["gpt_oss"]
    big = tables.layer_inputs(cfg, 512).x
    for T in cfg.t_sweep:
        assert np.array_equal(tables.layer_inputs(cfg, T).x, big[:T])


def test_zipf_shares_reported():
    tab = tables.load_table("midsize_zipf")
    got = np.array(tab["achieved_shares"])
    tgt = np.array(tab["target_shares"])
    assert abs(got.sum() - 1) < 1e-4
    assert np.all(np.diff(tgt) < 0) and got[0] > 0.25
    assert np.max(np.abs(got - tgt) / tgt) < 0.1


def test_config_shapes_match_page_parameter_counts():
    G = P.golden("parameter_counts.json")
    ds, go, mx = NAMED["deepseek_v3"], NAMED["gpt_oss"], NAMED["mixtral"]
    assert round(ds.expert_params() / 1e6, 0) == G["deepseek_expert_params_M"]
    assert round(G["deepseek_layers"] * G["deepseek_experts_per_layer"] * ds.expert_params() / 1e9,
                 1) == G["deepseek_total_expert_B"]
    assert round(G["deepseek_layers"] * (ds.k + ds.n_shared) * ds.expert_params() / 1e9,
                 1) == G["deepseek_active_expert_B"]
    assert round(G["gpt_oss_layers"] * go.E * go.expert_params() / 1e9, 1) == G["gpt_oss_moe_B"]
    exp_B = G["mixtral_layers"] * mx.E * mx.expert_params() / 1e9
    other = G["mixtral_total_B"] - exp_B
    assert round(other + exp_B * mx.k / mx.E, 1) == G["mixtral_active_B"]


def test_mx_weight_recipes():
    """MXFP4 and MXFP8 test weights: shapes, no NaN codes (MXFP8), a
    deterministic stream, and an rms within a factor of two of the dense
    recipe's 1/sqrt(fan_in)."""
    import oracle
    from moe_inputs import NAMED, generate
    cfg = NAMED["gpt_oss"]
    for fmt, draw, deq in (("mxfp4", generate.mxfp4_expert_weights, oracle.dequant_mxfp4),
                           ("mxfp8", generate.mxfp8_expert_weights, oracle.dequant_mxfp8)):
        (u, us), _, (d, ds) = draw(cfg, 3)
        assert u.shape == (cfg.ffn, cfg.d // (2 if fmt == "mxfp4" else 1)), fmt
        assert us.shape == (cfg.ffn, cfg.d // 32) and ds.shape == (cfg.d, cfg.ffn // 32)
        if fmt == "mxfp8":
            assert not np.isin(u, [0x7F, 0xFF]).any() and not np.isin(d, [0x7F, 0xFF]).any()
        (u2, _), _, _ = draw(cfg, 3)
        assert np.array_equal(u, u2)
        rms = float(np.sqrt(np.mean(deq(u, us) ** 2)))
        target = 1.0 / np.sqrt(cfg.d)
        assert target / 2 <= rms <= 2 * target, (fmt, rms, target)
