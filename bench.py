#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Headline workload: the Mixtral-shaped layer (d=4096, E=8, top-2, SwiGLU
ffn=14336, bf16 storage, fp32 accumulation) at T=4096 tokens (prefill).  One
step is one moe_forward over the whole batch (router, dispatch, both grouped
GEMMs, combine), inputs and weights already resident in HBM.

The same run times every other named layer and reports each under
"configs" with tokens/s and its roofline fraction: the Mixtral-shaped layer
at T=16 (decode), the mid-size Zipf layer at T=8192, the DeepSeek-V3-shaped
layer at T=4096 and the gpt-oss-shaped layer at T = 1, 8, 32, 128, 512.
Token rows, router weights and biases are the seeded, margin-filtered inputs
the parity tests use (they steer the routing); the expert weights of those
layers are filled on the device with seeded N(0, 1/fan_in) values, since
their values do not steer any kernel.

Prints ONE JSON line with the metric, the live roofline figure of the
dominant kernel (the up/gate grouped GEMM, timed with hipEvents recorded on
its launch stream inside the timed steps) and the fp64 CPU oracle's
throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec; grouped-GEMM % MFMA peak (prefill), % HBM peak (decode)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

# name -> (named layer, T, timing): "steps" = mean over back-to-back steps,
# "flushed" = median over iterations with L2 and MALL flushed in between
WORKLOADS = {
    "mixtral_t4096": ("mixtral", 4096, "steps"),
    "mixtral_t16": ("mixtral", 16, "flushed"),
    "midsize_zipf_t8192": ("midsize_zipf", 8192, "steps"),
    "deepseek_v3_t4096": ("deepseek_v3", 4096, "steps"),
    "gpt_oss_t1": ("gpt_oss", 1, "flushed"),
    "gpt_oss_t8": ("gpt_oss", 8, "flushed"),
    "gpt_oss_t32": ("gpt_oss", 32, "flushed"),
    "gpt_oss_t128": ("gpt_oss", 128, "flushed"),
    "gpt_oss_t512": ("gpt_oss", 512, "flushed"),
}
# The gpt-oss-shaped layer with MX-format experts (profiling runs only).
MX_WORKLOADS = {"mxfp4_gpt_oss_decode": "mxfp4", "mxfp8_gpt_oss_decode": "mxfp8"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-iters", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the T=16 decode leg")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the timed T=4096 steps (profiling the decode leg alone)")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MB",
                    help="also run one plain device copy of MB megabytes (a kernel of known "
                         "traffic, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens of the workload the CPU oracle runs")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle runs (median taken)")
    ap.add_argument("--workload", default="all",
                    help="'all' (default: the headline plus every config), or one of "
                         + ", ".join(WORKLOADS) + " to time that layer alone (for profiling), "
                         "or " + " / ".join(MX_WORKLOADS) + " for the gpt-oss-shaped layer "
                         "with MX-format experts at T = 1 ... 512")
    ap.add_argument("--variants", action="store_true",
                    help="also time the router options: sigmoid / raw routing on the "
                         "DeepSeek-V3-shaped router, capacity cuts on the Mixtral-shaped "
                         "layer, and MXFP4 and MXFP8 experts on the gpt-oss-shaped decode "
                         "layer (reported under \"variants\")")
    return ap.parse_args()


def upload_layer(cfg, T):
    import numpy as np
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from moe_inputs import generate, tables

    def dev(a):
        a = np.ascontiguousarray(a)
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(a).to("cuda")

    li = tables.layer_inputs(cfg, T)
    E = cfg.E
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    up = torch.empty((E, cfg.ffn, cfg.d), dtype=dt, device="cuda")
    gate = torch.empty_like(up)
    down = torch.empty((E, cfg.d, cfg.ffn), dtype=dt, device="cuda")
    for e, (u, g, dn) in generate.iter_experts(cfg, range(E)):
        up[e].copy_(dev(u))
        gate[e].copy_(dev(g))
        down[e].copy_(dev(dn))
    W = moe.Weights(w_router=dev(li.w_router), w_up=up, w_gate=gate, w_down=down,
                    bias=None if li.bias is None else torch.from_numpy(li.bias).cuda())
    return li, dev(li.x), W


def time_forward(x, W, k, steps, warmup):
    """K timed steps of the plain layer call bracketed by synchronize; then
    as many steps again, untimed by the wall clock, whose per-kernel
    durations come from the events each step records on its own launch
    stream (the records themselves cost a few microseconds per step, so they
    stay out of the timed steps)."""
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from sparse_mixture_experts_histogram_amd.hipevents import Events

    T = x.shape[0]
    desc = W.desc(T, k)
    ws = moe.workspace(desc, x.device)
    y = torch.empty((T, x.shape[1]), dtype=torch.float32, device=x.device)
    counts = torch.empty((W.w_up.shape[0],), dtype=torch.int32, device=x.device)
    ev = Events(6 * max(steps, 1))
    for _ in range(warmup):
        moe.moe_forward_timed(x, W, k, None, y, ws, counts=counts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_forward_timed(x, W, k, None, y, ws, counts=counts)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    for i in range(steps):
        moe.moe_forward_timed(x, W, k, ev.slice(6 * i, 6), y, ws, counts=counts)
    torch.cuda.synchronize()
    names = ["router", "dispatch", "expert_up", "expert_down", "combine"]
    per = {n: statistics.mean(ev.ms(6 * i + j, 6 * i + j + 1) for i in range(steps))
           for j, n in enumerate(names)}
    layer = statistics.mean(ev.ms(6 * i, 6 * i + 5) for i in range(steps))
    ev.close()
    return wall, layer, per, counts.cpu().numpy()


def time_decode(x, W, k, iters):
    """Per-iteration event timing with L2 and the 256 MB MALL flushed between
    iterations, outside the timed interval, by reading 1 GiB (a read leaves no
    dirty lines for the next kernel to write back); median.  The layer time
    comes from iterations that record events only before the first and after
    the last launch; the expert-GEMM time from a second set that records
    them between launches too."""
    import ctypes
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from sparse_mixture_experts_histogram_amd.hipevents import Events

    T = x.shape[0]
    ws = moe.workspace(W.desc(T, k), x.device)
    y = torch.empty((T, x.shape[1]), dtype=torch.float32, device=x.device)
    counts = torch.empty((W.w_up.shape[0],), dtype=torch.int32, device=x.device)
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=x.device)
    flush_sum = torch.empty((), dtype=torch.float32, device=x.device)
    ev = Events(6 * iters)
    outer = [(ctypes.c_void_p * 6)(ev.ev[6 * i], None, None, None, None, ev.ev[6 * i + 5])
             for i in range(iters)]
    for _ in range(5):
        moe.moe_forward_timed(x, W, k, None, y, ws, counts=counts)
    for i in range(iters):
        torch.sum(flush, dim=0, out=flush_sum)
        moe.moe_forward_timed(x, W, k, ctypes.cast(outer[i], ctypes.c_void_p), y, ws,
                              counts=counts)
    torch.cuda.synchronize()
    layer = statistics.median(ev.ms(6 * i, 6 * i + 5) for i in range(iters))
    for i in range(iters):
        torch.sum(flush, dim=0, out=flush_sum)
        moe.moe_forward_timed(x, W, k, ev.slice(6 * i, 6), y, ws, counts=counts)
    torch.cuda.synchronize()
    gemm = statistics.median(ev.ms(6 * i + 2, 6 * i + 4) for i in range(iters))
    ev.close()
    del flush
    return layer, gemm, counts.cpu().numpy()


def decode_leg(cfg, x, W, k, iters):
    import numpy as np
    xd = x[:16].contiguous()
    dec_layer, dec_gemm, dec_counts = time_decode(xd, W, k, iters)
    touched = int(np.sum(dec_counts > 0))
    touched_bytes = touched * 3 * cfg.d * cfg.ffn * 2
    fig = layer_figures(cfg, 16, dec_layer, dec_counts)
    fig["expert_gemms_ms"] = round(dec_gemm, 4)
    fig["grouped_gemm_hbm_frac"] = round(touched_bytes / (dec_gemm * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)
    fig["timing"] = (f"median of {iters} hipEvent-timed layers, L2 and MALL flushed between them")
    dec = {"T": 16, "ms_per_step": round(dec_layer, 4), "tokens_per_s": round(16 / dec_layer * 1e3, 1),
           "experts_touched": touched, "touched_weight_bytes": touched_bytes,
           "hbm_frac_layer": round(touched_bytes / (dec_layer * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
           "hbm_frac_expert_gemms": round(touched_bytes / (dec_gemm * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
           "timing": "median of per-iteration hipEvent times (events before the first and after the "
                     "last launch only), L2 and MALL flushed by a 1 GiB read between iterations",
           "figures": fig}
    return dec


def time_variants(cfg, x, W, k, steps):
    """Router options, timed with events on the launch stream (mean of
    `steps` calls after 5 warm-up calls each):

    * moe_route on the DeepSeek-V3-shaped router (T=4096, d=7168, E=256,
      top-8, bias ~ N(0, 0.5)) with softmax, sigmoid and raw-weight scoring;
      bytes are x and W_r read once plus the indices and weights written;
    * the whole Mixtral-shaped T=4096 layer with capacity factors 1.0 and
      1.25 (the dropless layer is the headline), with the dropped pairs;
    * the gpt-oss-shaped layer with MXFP4 experts at decode batch sizes."""
    import numpy as np
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from moe_inputs import NAMED, generate, tables

    def ev_time(fn):
        for _ in range(5):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    out = {}
    ds = NAMED["deepseek_v3"]
    T = 4096
    li = tables.layer_inputs(ds, T)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    xd = bf(li.x)
    # expert weights are not read by the router: uninitialised storage of the right shape
    Wd = moe.Weights(w_router=bf(generate.router_weight(ds)),
                     w_up=torch.empty((ds.E, ds.ffn, ds.d), dtype=torch.bfloat16, device="cuda"),
                     w_gate=torch.empty((ds.E, ds.ffn, ds.d), dtype=torch.bfloat16, device="cuda"),
                     w_down=torch.empty((ds.E, ds.d, ds.ffn), dtype=torch.bfloat16, device="cuda"),
                     bias=torch.from_numpy(generate.normal_bias(ds)).cuda())
    ws = moe.workspace(Wd.desc(T, ds.k), xd.device)
    rbytes = T * ds.d * 2 + ds.E * ds.d * 2 + T * ds.k * 8
    router = {}
    for name, rt in (("softmax", moe.Routing()), ("sigmoid", moe.Routing(scoring="sigmoid")),
                     ("sigmoid_raw", moe.Routing(scoring="sigmoid", renormalize=False)),
                     ("softmax_raw", moe.Routing(renormalize=False))):
        ms = ev_time(lambda: moe.moe_route(xd, Wd, ds.k, ws=ws, routing=rt))
        router[name] = {"us": round(ms * 1e3, 2),
                        "hbm_frac": round(rbytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}
    out["router_deepseek_v3_t4096"] = {"algorithmic_bytes": rbytes, **router}
    del xd, Wd, ws
    torch.cuda.empty_cache()

    Tm = x.shape[0]
    cap_out = {}
    for f in (1.0, 1.25):
        rt = moe.Routing(capacity_factor=f)
        wsm = moe.workspace(W.desc(Tm, k, routing=rt), x.device)
        ms = ev_time(lambda: moe.moe_forward(x, W, k, ws=wsm, routing=rt))
        _, _, _, counts = moe.moe_forward(x, W, k, ws=wsm, routing=rt, return_routing=True)
        cnt = counts.cpu().numpy()
        cap = int(np.ceil(Tm * k / cfg.E * f))
        cap_out[str(f)] = {"ms": round(ms, 4), "tokens_per_s": round(Tm / ms * 1e3, 1),
                           "capacity": cap, "dropped_pairs": int(np.clip(cnt - cap, 0, None).sum())}
        del wsm
    out["capacity_mixtral_t4096"] = cap_out
    out["mxfp4_gpt_oss_decode"] = time_mx_decode([1, 8, 32, 128, 512], 50)
    out["mxfp8_gpt_oss_decode"] = time_mx_decode([1, 8, 32, 128, 512], 50, fmt="mxfp8")
    out["mxfp4_gpt_oss_decode_line_rows"] = time_mx_decode([1, 8, 32, 128, 512], 50,
                                                           line_rows=True)
    out["mxfp8_gpt_oss_decode_line_rows"] = time_mx_decode([1, 8, 32, 128, 512], 50,
                                                           fmt="mxfp8", line_rows=True)
    return out


def time_mx_decode(Ts, iters, fmt="mxfp4", line_rows=False):
    """The gpt-oss-shaped layer (d=2880, 128 experts, top-4, ffn 2880) with
    MXFP4 (or, fmt="mxfp8", MXFP8) expert weights at decode batch sizes:
    per-iteration hipEvents before the first and after the last launch, L2
    and MALL flushed by a 1 GiB read between iterations, median of `iters`;
    HBM fraction on the touched experts' code and scale bytes.  line_rows:
    code rows padded to whole 128-byte lines (MOE_FLAG_MX_LINE_ROWS; the
    fraction still counts the codes' own bytes)."""
    import ctypes
    import numpy as np
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from sparse_mixture_experts_histogram_amd.hipevents import Events
    from moe_inputs import NAMED, generate, tables

    cfg = NAMED["gpt_oss"]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def tc(a):  # code rows, padded to whole lines with line_rows
        if not line_rows:
            return t(a)
        R = a.shape[-1]
        out = np.zeros(a.shape[:-1] + ((R + 127) // 128 * 128,), dtype=np.uint8)
        out[..., :R] = a
        return t(out)

    stack = generate.stacked_mxfp4 if fmt == "mxfp4" else generate.stacked_mxfp8
    u, us, g, gs, dn, ds = stack(cfg)
    li = tables.layer_inputs(cfg, max(Ts))
    W = moe.MxWeights(w_router=torch.from_numpy(li.w_router.view(np.int16)).view(torch.bfloat16).cuda(),
                      up=tc(u), up_scale=t(us), gate=tc(g), gate_scale=t(gs), down=tc(dn),
                      down_scale=t(ds), line_rows=line_rows, expert_format=fmt)
    del u, us, g, gs, dn, ds
    xall = torch.from_numpy(li.x.view(np.int16)).view(torch.bfloat16).cuda()
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    flush_sum = torch.empty((), dtype=torch.float32, device="cuda")
    per_expert = 3 * cfg.d * cfg.ffn * ((0.5 if fmt == "mxfp4" else 1.0) + 1.0 / 32)
    res = {}
    for T in Ts:
        x = xall[:T].contiguous()
        ws = moe.workspace(W.desc(T, cfg.k), x.device)
        y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
        ev = Events(6 * iters)
        outer = [(ctypes.c_void_p * 6)(ev.ev[6 * i], None, None, None, None, ev.ev[6 * i + 5])
                 for i in range(iters)]
        for _ in range(5):
            moe.moe_forward_mx(x, W, cfg.k, ws=ws, y=y)
        for i in range(iters):
            torch.sum(flush, dim=0, out=flush_sum)
            moe.moe_forward_mx(x, W, cfg.k, ws=ws, y=y,
                               events=ctypes.cast(outer[i], ctypes.c_void_p))
        torch.cuda.synchronize()
        ms = statistics.median(ev.ms(6 * i, 6 * i + 5) for i in range(iters))
        ev.close()
        _, _, _, counts = moe.moe_forward_mx(x, W, cfg.k, ws=ws, return_routing=True)
        touched = int((counts > 0).sum())
        res[str(T)] = {"ms": round(ms, 4), "tokens_per_s": round(T / ms * 1e3, 1),
                       "experts_touched": touched,
                       "hbm_frac": round(touched * per_expert / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}
    del flush
    return res


def kernel_source_hash() -> str:
    """Hash of the expert-GEMM kernel source the library was built from."""
    import hashlib
    p = os.path.join(ROOT, "sparse_mixture_experts_histogram_amd", "csrc", "experts.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(key):
    """HBM bytes per launch of a kernel from the stored rocprofv3 counter
    record (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or
    None when the record is missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("experts_hip_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, li, sample, reps):
    """The fp64 oracle as written, on the first `sample` tokens of the same
    workload (routing and every chosen expert), median of `reps` runs."""
    import oracle
    from moe_inputs import generate
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    xs = li.x[:sample]
    # the weights are inputs: drawn outside the timed region
    wts = {e: generate.expert_weights(cfg, e) for e in range(cfg.E)}
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.moe_forward(xs, li.w_router, li.bias, cfg.k, lambda e: wts[e], cfg.E, cfg.dtype)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    info = host_info()
    return {"value": round(sample / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": info["cpu"], "blas": info["blas"],
            "sample": f"first {sample} tokens of the {cfg.name} T={cfg.T} workload (routing + "
                      f"chosen experts), fp64 numpy oracle, median of {reps} runs of "
                      f"{dt:.2f} s each ({sum(times):.1f} s total)"}


def upload_routing_inputs(cfg, T, seed=1234):
    """Seeded, margin-filtered token rows, router weight and bias of a named
    layer (what steers the routing), and expert weights filled on the device
    with N(0, 1/fan_in) values from a seeded torch generator."""
    import numpy as np
    import torch
    import sparse_mixture_experts_histogram_amd as moe
    from moe_inputs import tables

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    li = tables.layer_inputs(cfg, T)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + cfg.config_id)

    def fill(n, rows, cols):
        out = torch.empty((n, rows, cols), dtype=torch.bfloat16, device="cuda")
        for e in range(n):  # one matrix at a time: no large float32 temporary
            out[e].copy_(torch.randn((rows, cols), generator=g, device="cuda")
                         .mul_(1.0 / cols ** 0.5))
        return out

    W = moe.Weights(w_router=dev(li.w_router), w_up=fill(cfg.E, cfg.ffn, cfg.d),
                    w_gate=fill(cfg.E, cfg.ffn, cfg.d), w_down=fill(cfg.E, cfg.d, cfg.ffn),
                    bias=None if li.bias is None else torch.from_numpy(li.bias).cuda())
    if cfg.n_shared:
        W.ws_up = fill(cfg.n_shared, cfg.ffn_shared, cfg.d)
        W.ws_gate = fill(cfg.n_shared, cfg.ffn_shared, cfg.d)
        W.ws_down = fill(cfg.n_shared, cfg.d, cfg.ffn_shared)
    return li, dev(li.x), W


def layer_figures(cfg, T, ms, counts, per=None):
    """tokens/s and roofline fractions of one layer time.  Algorithmic FLOPs:
    2*T*d*E for the router plus 2 per weight per (token, expert) pair (the
    shared experts included).  Bytes: the touched experts' weights (an expert
    with at least one pair, and every shared expert), the router matrix, x,
    y in fp32 and the routing indices and weights; padding and the
    intermediates h and expert outputs are implementation traffic and are not
    counted."""
    import numpy as np
    eb = cfg.elem_bytes
    touched = int(np.sum(np.asarray(counts) > 0))
    w_bytes = (touched * 3 * cfg.d * cfg.ffn + cfg.n_shared * 3 * cfg.d * cfg.ffn_shared) * eb
    alg_bytes = (w_bytes + cfg.E * cfg.d * eb + T * cfg.d * eb + T * cfg.d * 4 + T * cfg.k * 8)
    flops = cfg.flops(T)
    out = {"T": T, "ms": round(ms, 4), "tokens_per_s": round(T / ms * 1e3, 1),
           "experts_touched": touched, "touched_weight_bytes": w_bytes,
           "algorithmic_bytes": alg_bytes, "algorithmic_flops": flops,
           "hbm_frac_touched_weights": round(w_bytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
           "hbm_frac_algorithmic": round(alg_bytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
           "mfma_frac": round(flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)}
    if per is not None:
        out["kernels_ms"] = {n: round(v, 4) for n, v in per.items()}
        pairs = T * cfg.k
        f_up = 4.0 * cfg.d * (cfg.ffn * pairs + cfg.ffn_shared * T * cfg.n_shared)
        out["grouped_gemm_mfma_frac"] = round(
            1.5 * f_up / ((per["expert_up"] + per["expert_down"]) * 1e-3)
            / (PEAK_BF16_TFLOPS * 1e12), 4)
        out["grouped_gemm_hbm_frac"] = round(
            w_bytes / ((per["expert_up"] + per["expert_down"]) * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)
    return out


def run_workload(name, steps, warmup, iters):
    """Time one named workload on device-filled expert weights."""
    import torch
    from moe_inputs import NAMED
    layer, T, how = WORKLOADS[name]
    cfg = NAMED[layer]
    t0 = time.perf_counter()
    li, x, W = upload_routing_inputs(cfg, T)
    torch.cuda.synchronize()
    t_in = time.perf_counter() - t0
    if how == "steps":
        wall, _, per, counts = time_forward(x, W, cfg.k, steps, warmup)
        fig = layer_figures(cfg, T, wall * 1e3, counts, per)
        fig["timing"] = f"mean of {steps} back-to-back steps (wall clock), per-kernel hipEvents"
    else:
        ms, gemm, counts = time_decode(x, W, cfg.k, iters)
        fig = layer_figures(cfg, T, ms, counts)
        fig["expert_gemms_ms"] = round(gemm, 4)
        fig["grouped_gemm_hbm_frac"] = round(fig["touched_weight_bytes"] / (gemm * 1e-3)
                                             / (PEAK_HBM_GBS * 1e9), 4)
        fig["timing"] = (f"median of {iters} hipEvent-timed layers, L2 and MALL flushed "
                         "between them")
    print(f"[bench] {name}: {fig} (inputs {t_in:.1f}s)", file=sys.stderr, flush=True)
    del x, W, li
    torch.cuda.empty_cache()
    return fig


def copy_check(mb):
    """One elementwise kernel that reads and writes exactly `mb` megabytes
    (after a fill that writes them): a kernel of known traffic for scaling
    rocprofv3's FETCH_SIZE and WRITE_SIZE."""
    import torch
    n = mb * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def host_info():
    """CPU model, visible cores and the BLAS numpy calls."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return {"cpu": model, "cores_visible": len(os.sched_getaffinity(0)), "blas": blas}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU expert parallelism is not implemented; the library runs one GPU)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from moe_inputs import NAMED

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_check:
        copy_check(args.copy_check)
    if args.workload in MX_WORKLOADS:
        res = time_mx_decode(list(NAMED["gpt_oss"].t_sweep), args.decode_iters,
                             fmt=MX_WORKLOADS[args.workload])
        print(json.dumps({"workload": args.workload, "T": res}), flush=True)
        return
    if args.workload != "all":
        if args.workload not in WORKLOADS:
            sys.exit(f"bench.py: unknown workload {args.workload}; one of "
                     f"{', '.join(list(WORKLOADS) + list(MX_WORKLOADS))}")
        fig = run_workload(args.workload, args.steps, args.warmup, args.decode_iters)
        print(json.dumps({"workload": args.workload, **fig}), flush=True)
        return

    cfg = NAMED["mixtral"]
    T, k = 4096, cfg.k
    t_in = time.perf_counter()
    li, x, W = upload_layer(cfg, T)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_in:.1f}s", file=sys.stderr,
          flush=True)

    if args.no_prefill:
        dec = decode_leg(cfg, x, W, k, args.decode_iters)
        print(json.dumps({"decode_only": dec}), flush=True)
        return
    wall, layer, per, counts = time_forward(x, W, k, args.steps, args.warmup)
    print(f"[bench] prefill: {wall * 1e3:.3f} ms/step wall, per-kernel ms {per}",
          file=sys.stderr, flush=True)
    flops_up = 4.0 * cfg.d * cfg.ffn * T * k
    flops_down = 2.0 * cfg.d * cfg.ffn * T * k
    flops_layer = cfg.flops(T)
    up_tf = flops_up / (per["expert_up"] * 1e-3) / 1e12
    down_tf = flops_down / (per["expert_down"] * 1e-3) / 1e12
    gemm_tf = (flops_up + flops_down) / ((per["expert_up"] + per["expert_down"]) * 1e-3) / 1e12

    configs = {"mixtral_t4096": layer_figures(cfg, T, wall * 1e3, counts, per)}
    configs["mixtral_t4096"]["timing"] = "the headline steps (wall clock), per-kernel hipEvents"
    # decode leg: same layer and weights, first 16 tokens
    dec = None
    if not args.no_decode:
        dec = decode_leg(cfg, x, W, k, args.decode_iters)
        print(f"[bench] decode: {dec}", file=sys.stderr, flush=True)
        configs["mixtral_t16"] = dec.pop("figures")

    variants = None
    if args.variants:
        variants = time_variants(cfg, x, W, k, args.steps)
        print(f"[bench] variants: {variants}", file=sys.stderr, flush=True)
    del x, W
    torch.cuda.empty_cache()

    for name in WORKLOADS:
        if name.startswith("mixtral"):
            continue
        configs[name] = run_workload(name, min(args.steps, 20), min(args.warmup, 5),
                                     args.decode_iters)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, li, args.cpu_sample, args.cpu_reps)
        print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC, "value": round(T / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": "mixtral_prefill", "T": T, "d": cfg.d, "E": cfg.E, "k": k,
                   "ffn": cfg.ffn, "n_shared": 0, "storage": "bf16", "accumulate": "fp32",
                   "y": "fp32", "path": "prefill", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "expert_up (grouped up/gate GEMM + SwiGLU)",
                     "achieved": round(up_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(up_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic("expert_up_mixtral_t4096"),
                     "traffic_source": "stored rocprofv3 FETCH_SIZE + WRITE_SIZE record "
                                       "(profiles/traffic.json), null unless taken on this "
                                       "kernel source",
                     "avg_launch_ms": round(per["expert_up"], 4),
                     "algorithmic_flops_per_launch": flops_up},
        "grouped_gemm": {"frac_mfma": round(gemm_tf / PEAK_BF16_TFLOPS, 4),
                         "up_frac_mfma": round(up_tf / PEAK_BF16_TFLOPS, 4),
                         "down_frac_mfma": round(down_tf / PEAK_BF16_TFLOPS, 4),
                         "down_traffic": stored_traffic("expert_down_mixtral_t4096")},
        "grouped_gemm_frac_mfma": round(gemm_tf / PEAK_BF16_TFLOPS, 4),
        "layer_tflops": round(flops_layer / (layer * 1e-3) / 1e12, 2),
        "kernels_ms": {kname: round(v, 4) for kname, v in per.items()},
        "expert_counts": [int(c) for c in counts],
        "decode": dec,
        "configs": configs,
        "cpu_baseline": cpu,
        **({"variants": variants} if variants is not None else {}),
        "host": host_info(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
