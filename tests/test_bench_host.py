"""Host-side parts of bench.py (no GPU): the one-GPU guard, the stored
traffic record's source check, and the layer figures' formulas."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_inputs import NAMED  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_only_for_its_kernel_source(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)["expert_up_mixtral_t4096"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["experts_hip_sha256_16"])
    assert bench.stored_traffic("expert_up_mixtral_t4096") == rec["bytes_per_launch"]
    # the record is the scaled sum of the two counter passes
    assert rec["bytes_per_launch"] == rec["read_bytes"] + rec["write_bytes"]
    assert abs(rec["read_bytes"] - rec["fetch_size_kib"] * 1024 * rec["fetch_factor"]) < 1e-3 * rec["read_bytes"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic("expert_up_mixtral_t4096") is None
    assert bench.stored_traffic("no_such_kernel") is None


def test_layer_figures_formulas():
    cfg = NAMED["mixtral"]
    T, ms = 4096, 2.5
    counts = np.array([1000, 0, 1200, 1000, 1000, 1000, 1000, 2992])  # 7 experts touched
    fig = bench.layer_figures(cfg, T, ms, counts)
    w_bytes = 7 * 3 * cfg.d * cfg.ffn * 2
    assert fig["experts_touched"] == 7
    assert fig["touched_weight_bytes"] == w_bytes
    assert abs(fig["hbm_frac_touched_weights"] - w_bytes / (ms * 1e-3) / 8e12) < 1e-4
    assert abs(fig["tokens_per_s"] - T / ms * 1e3) < 0.1
    flops = 2 * T * cfg.d * cfg.E + 6 * cfg.d * cfg.ffn * T * cfg.k
    assert fig["algorithmic_flops"] == flops
    assert abs(fig["mfma_frac"] - flops / (ms * 1e-3) / 2.5e15) < 1e-4
