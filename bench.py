#!/usr/bin/env python3
"""Benchmark of the MS-GLA layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main]

One step = one msgla_forward (pool+projection GEMM, chunk-local GLA kernel,
chunk-state GLA kernel, hold+fusion+output-projection GEMM) over the whole
batch, inputs and packed weights already resident in HBM.  W untimed warm-up
steps, then K timed steps bracketed by device synchronisation; per-stage
durations come from HIP events the library records on the same stream inside
the timed region.  The single-scale GLA layer (4 heads at scale 1, same
shapes) is timed the same way for the ratio.  The fp64 CPU oracle is timed on
the host on a bounded sample of the same workload.  Prints one JSON line.

Inputs are seeded synthetic Gaussians (see scale_gla_layer_amd/synth.py);
the workloads of the MS-GLA notes were trained-model runs on FineWeb-Edu, and
the layer's cost does not depend on data values.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0}
STAGES = ("pool_proj", "gla_chunk", "gla_state", "hold_fuse")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(cfg, B, L):
    """Algorithmic flops and bytes of the layer and of each stage.

    Flops: projections 2 T d (h(2dk+dv)+r), gate 2 T r h dk, GLA core
    T h (4 dk dv + (C+1)(dk+dv)) per pooled token T, output projection at the
    coarse length 2 T h dv d, fusion logits 2 B L d m.  Bytes: x, out and the
    weights once (storage type), the GLA core's q/k/v/g in and y out."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, dk, dv, r, C = cfg.d_model, cfg.d_k, cfg.d_v, cfg.gate_rank, cfg.chunk
    m = len(cfg.scales)
    f_proj = f_gate = f_scan = f_out = 0.0
    w_bytes = 0.0
    core_bytes = 0.0
    for s, h in zip(cfg.scales, cfg.heads):
        T = B * (L // s)
        f_proj += 2.0 * T * d * (h * (2 * dk + dv) + r)
        f_gate += 2.0 * T * r * h * dk
        f_scan += float(T) * h * (4 * dk * dv + (C + 1) * (dk + dv))
        f_out += 2.0 * T * h * dv * d
        w_bytes += es * (d * (h * (2 * dk + dv) + r) + r * h * dk + h * dv * d) + 4 * h * dk
        core_bytes += T * (h * (2 * dk + 2 * dv) * es + r * 4)
    f_fuse = 2.0 * B * L * d * m if m > 1 else 0.0
    w_bytes += es * d * m if m > 1 else 0
    io_bytes = 2.0 * B * L * d * es
    return {
        "flops": f_proj + f_gate + f_scan + f_out + f_fuse,
        "bytes": io_bytes + w_bytes,
        "stage": {
            "pool_proj": ("mfma", f_proj + f_fuse),
            "gla_chunk": ("hbm", core_bytes),
            "gla_state": ("hbm", core_bytes),
            "hold_fuse": ("mfma", f_out),
        },
    }


def time_forward(layer, x, steps, warmup, events_per_step=True):
    import torch
    B, L, _ = x.shape
    out = layer.new_output(B, L)
    for _ in range(warmup):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in STAGES] for _ in range(steps)]
    for row in ev:  # materialise the HIP events before handing them to the library
        for a, b in row:
            a.record()
            b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        if events_per_step:
            layer.forward(x, out=out, events=([a for a, _ in ev[k]], [b for _, b in ev[k]]))
        else:
            layer.forward(x, out=out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)]))
                for i, name in enumerate(STAGES)} if events_per_step else {}
    return dt / steps * 1e3, stage_ms


def cpu_baseline(cfg, X, W, budget_s=12.0):
    from oracle import msgla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, L, _ = X.shape
    done, t0 = 0, time.perf_counter()
    while done < B and (time.perf_counter() - t0) < budget_s:
        orc.layer_forward(X[done: done + 1], W, cfg)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done * L / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {B} sequences x {L} tokens of the same workload "
                      f"({dt:.1f} s; fp64 NumPy, token-by-token recurrence; "
                      f"BLAS threads {threads}, the recurrence loop itself is single-threaded)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gla", action="store_true", help="skip the single-scale GLA comparison")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this layer's path is built and timed on a single "
              f"MI355X); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from scale_gla_layer_amd.synth import make_inputs

    wl = WORKLOADS[args.workload]
    cfg, B, L = wl.cfg, wl.batch, wl.seq_len
    log(f"[bench] workload {wl.name}: {wl.description}")
    X, W = make_inputs(cfg, B, L, seed=0, gate_bias=wl.gate_bias)
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    ms, stage_ms = time_forward(layer, x, args.steps, args.warmup)
    tok_s = B * L / (ms * 1e-3)
    log(f"[bench] {ms * 1e3:.1f} us/step, {tok_s / 1e6:.1f} M tokens/s; stages (us): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in stage_ms.items()))

    alg = algorithmic(cfg, B, L)
    peak_f = PEAK["bf16_mfma_tflops"] if cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
    layer_tflops = alg["flops"] / (ms * 1e-3) / 1e12
    t_roof = max(alg["flops"] / (peak_f * 1e12), alg["bytes"] / (PEAK["hbm_gbs"] * 1e9))
    dom = max(stage_ms, key=stage_ms.get)
    bound, amount = alg["stage"][dom]
    dur = stage_ms[dom] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = amount / dur / 1e12, peak_f, "TFLOP/s"
    else:
        achieved, peak, unit = amount / dur / 1e9, PEAK["hbm_gbs"], "GB/s"
    stages = {}
    for name, t in stage_ms.items():
        b, a = alg["stage"][name]
        rate = a / (t * 1e-3) / (1e12 if b == "mfma" else 1e9)
        stages[name] = {"us": round(t * 1e3, 2), "bound": b,
                        "achieved": round(rate, 1), "unit": "TFLOP/s" if b == "mfma" else "GB/s",
                        "frac": round(rate / (peak_f if b == "mfma" else PEAK["hbm_gbs"]), 4)}

    ratio_vs_gla = None
    gla = None
    if not args.no_gla and args.workload != "gla_baseline":
        gwl = WORKLOADS["gla_baseline"]
        Xg, Wg = make_inputs(gwl.cfg, gwl.batch, gwl.seq_len, seed=0)
        glayer = DeviceLayer(gwl.cfg, Wg)
        xg = to_device(Xg, gwl.cfg.dtype)
        gms, _ = time_forward(glayer, xg, args.steps, args.warmup, events_per_step=False)
        gla = gwl.batch * gwl.seq_len / (gms * 1e-3)
        ratio_vs_gla = tok_s / gla
        log(f"[bench] GLA baseline {gms * 1e3:.1f} us/step, {gla / 1e6:.1f} M tokens/s; "
            f"ratio {ratio_vs_gla:.3f}")
        del glayer, xg

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on the host ...")
        cpu = cpu_baseline(cfg, X, W)
        log(f"[bench] oracle {cpu['value']:.0f} tokens/s ({cpu['sample']})")

    line = {
        "metric": "MS-GLA layer fwd tokens/sec (B=8,L=2048,d=1024,bf16); % roofline; ratio vs GLA",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian inputs and weights)",
        "config": {"workload": wl.name, "batch": B, "seq_len": L, "d_model": cfg.d_model,
                   "scales": list(cfg.scales), "heads": list(cfg.heads), "d_k": cfg.d_k,
                   "d_v": cfg.d_v, "gate_rank": cfg.gate_rank, "chunk": cfg.chunk},
        "roofline": {"bound": bound, "kernel": dom, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": None},
        "layer_roofline": {"algorithmic_gflop": round(alg["flops"] / 1e9, 2),
                           "algorithmic_mb": round(alg["bytes"] / 1e6, 2),
                           "achieved_tflops": round(layer_tflops, 1),
                           "t_roof_us": round(t_roof * 1e6, 2),
                           "frac": round(t_roof / (ms * 1e-3), 4)},
        "stages": stages,
        "ratio_vs_gla": None if ratio_vs_gla is None else round(ratio_vs_gla, 4),
        "gla_tokens_per_s": None if gla is None else round(gla, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
