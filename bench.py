#!/usr/bin/env python3
"""Benchmark of the MS-GLA layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main]

One step = one msgla_forward (pooling prepass, projection GEMM, chunk-local
GLA kernel, chunk-state GLA kernel, hold+fusion+output-projection GEMM) over
the whole batch, inputs and packed weights already resident in HBM.  W untimed
warm-up steps, then K timed steps bracketed by device synchronisation;
per-kernel durations come from HIP events the library records on its own
stream inside the timed region.  The single-scale GLA layer (4 heads at scale
1, same shapes) is timed the same way for the ratio.  The fp64 CPU oracle is
timed on the host on a bounded sample of the same workload.  Prints one JSON
line.

Inputs are seeded synthetic Gaussians (see scale_gla_layer_amd/synth.py);
the workloads of the MS-GLA notes were trained-model runs on FineWeb-Edu, and
the layer's cost does not depend on data values.

    python bench.py --copy-calibration

runs only a plain 256 MiB device copy (the reference kernel for scaling the
FETCH_SIZE / WRITE_SIZE counters to bytes) and prints nothing else.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0}
# stage i of msgla_forward_timed and the kernel it times
STAGES = ("pool", "proj", "gla_chunk", "gla_state", "out_coarse", "hold_fuse")
KERNELS = {"pool": "k_pool", "proj": "k1_pool_proj", "gla_chunk": "k2a_gla_chunk",
           "gla_state": "k2b_gla_state", "out_coarse": "k3c_coarse", "hold_fuse": "k3f_fine_fuse"}
# sources a kernel's code depends on (a committed counter summary is only used
# while these are unchanged)
KERNEL_SOURCES = {
    "k1_pool_proj": ["k_pool_proj.hip", "gemm_dma.hpp", "async_copy.hpp", "device_common.hpp",
                     "layout.hpp"],
    "k3c_coarse": ["k_hold_fuse.hip", "gemm_dma.hpp", "async_copy.hpp", "device_common.hpp",
                   "layout.hpp"],
    "k3f_fine_fuse": ["k_hold_fuse.hip", "gemm_dma.hpp", "async_copy.hpp", "device_common.hpp",
                      "layout.hpp"],
    "k2a_gla_chunk": ["k_gla_chunk.hip", "device_common.hpp", "layout.hpp"],
    "k2b_gla_state": ["k_gla_state.hip", "async_copy.hpp", "device_common.hpp", "layout.hpp"],
    "k_pool": ["k_pool.hip", "device_common.hpp", "layout.hpp"],
}
COPY_CAL_BYTES = 256 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "scale_gla_layer_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic(cfg, B, L):
    """Algorithmic flops and bytes of the layer and of each kernel.

    Flops: projections 2 T d (h(2dk+dv)+r), gate 2 T r h dk, GLA core
    T h (4 dk dv + (C+1)(dk+dv)) per pooled token T, output projection at the
    coarse length 2 T h dv d, fusion logits 2 B L d m.  Layer bytes: x, out
    and the weights once (storage type).  Per kernel: the pooling prepass
    reads x and writes the block means; the GLA core moves q, k, v, the gate
    factor and y once (split as q, k, g into the chunk-local kernel and v, y
    through the state kernel); the GEMMs are counted by their flops (the
    output projections split into the coarse branches and the scale-1
    branch, whose GEMM carries the hold and fusion)."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, dk, dv, r, C = cfg.d_model, cfg.d_k, cfg.d_v, cfg.gate_rank, cfg.chunk
    m = len(cfg.scales)
    f_proj = f_gate = f_scan = f_out = f_out_coarse = 0.0
    fuse_bytes = 2.0 * B * L * d * es if len(cfg.scales) > 1 else 0.0
    w_bytes = 0.0
    chunk_bytes = state_bytes = 0.0
    pool_bytes = 0.0
    for s, h in zip(cfg.scales, cfg.heads):
        T = B * (L // s)
        f_proj += 2.0 * T * d * (h * (2 * dk + dv) + r)
        f_gate += 2.0 * T * r * h * dk
        f_scan += float(T) * h * (4 * dk * dv + (C + 1) * (dk + dv))
        f_out += 2.0 * T * h * dv * d
        if s > 1:
            f_out_coarse += 2.0 * T * h * dv * d
            fuse_bytes += T * d * es
        w_bytes += es * (d * (h * (2 * dk + dv) + r) + r * h * dk + h * dv * d) + 4 * h * dk
        chunk_bytes += T * (h * 2 * dk * es + r * 4)
        state_bytes += T * h * 2 * dv * es
        if s > 1:
            pool_bytes += T * d * es
    if pool_bytes:
        pool_bytes += B * L * d * es
    f_fuse = 2.0 * B * L * d * m if m > 1 else 0.0
    w_bytes += es * d * m if m > 1 else 0
    io_bytes = 2.0 * B * L * d * es
    return {
        "flops": f_proj + f_gate + f_scan + f_out + f_fuse,
        "bytes": io_bytes + w_bytes,
        "stage": {
            "pool": ("hbm", pool_bytes),
            "proj": ("mfma", f_proj + f_fuse),
            "gla_chunk": ("hbm", chunk_bytes),
            "gla_state": ("hbm", state_bytes),
            "out_coarse": ("mfma", f_out_coarse),
            # the scale-1 projection if there is one, else the hold + fusion traffic
            "hold_fuse": ("mfma", f_out - f_out_coarse) if f_out > f_out_coarse else
                         ("hbm", fuse_bytes),
        },
    }


def decode_algorithmic_bytes(cfg, B):
    """Average HBM bytes of one decode step: a branch of scale s completes a
    block on one step in s, and then reads its projection weights (q, k, v
    and the gate's first factor), the gate's second factor, W_o, and reads and
    writes its fp32 state; every step every branch reads and writes its fp32
    pending sum and reads or writes its fp32 held output; x_t, out_t and the
    fusion weights are read or written once."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, dk, dv, r = cfg.d_model, cfg.d_k, cfg.d_v, cfg.gate_rank
    m = len(cfg.scales)
    total = 2.0 * B * d * es + (d * m * es if m > 1 else 0)
    for s, h in zip(cfg.scales, cfg.heads):
        block = (es * d * (h * (2 * dk + dv) + r) + 4 * (r * h * dk + h * dk) + es * h * dv * d
                 + 2.0 * 4 * B * h * dk * dv)
        total += block / s + 3.0 * 4 * B * d
    return total


def measure_decode(workload="sweep_1248", steps=256, warmup=32):
    """Streaming decode: prefill the workload's sequences, then time `steps`
    back-to-back msgla_decode_step calls (HIP events around the loop)."""
    import time
    import torch
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from scale_gla_layer_amd.synth import make_inputs
    wl = WORKLOADS[workload]
    B, L0 = wl.batch, wl.seq_len
    X, W = make_inputs(wl.cfg, B, L0 + warmup + steps, seed=0)
    layer = DeviceLayer(wl.cfg, W)
    st = layer.new_state(B)
    layer.forward(to_device(X[:, :L0], wl.cfg.dtype), state_out=st)
    xs = [to_device(np.ascontiguousarray(X[:, t]), wl.cfg.dtype) for t in range(L0, L0 + warmup + steps)]
    out = layer.decode_step(xs[0], st)
    for t in range(1, warmup):
        layer.decode_step(xs[t], st, out_t=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        layer.decode_step(xs[t], st, out_t=out)
    h1 = time.perf_counter()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the same steps replayed from one captured HIP graph (token copied in each step)
    from scale_gla_layer_amd.runner import DecodeGraph
    st2 = layer.new_state(B)
    layer.forward(to_device(X[:, :L0], wl.cfg.dtype), state_out=st2)
    g = DecodeGraph(layer, st2, B)
    for t in range(warmup):
        g.step(xs[t])
    torch.cuda.synchronize()
    e0.record()
    for t in range(warmup, warmup + steps):
        g.step(xs[t])
    e1.record()
    torch.cuda.synchronize()
    us_g = e0.elapsed_time(e1) * 1e3 / steps
    alg = decode_algorithmic_bytes(wl.cfg, B)
    return {"workload": workload, "batch": B, "prefill": L0, "steps": steps,
            "us_per_step": round(us, 2), "tokens_per_s": round(B / (us * 1e-6), 1),
            "us_per_step_graph": round(us_g, 2),
            "host_us_per_call": round((h1 - h0) * 1e6 / steps, 2),
            "algorithmic_mb_per_step": round(alg / 1e6, 2),
            "achieved_gb_s": round(alg / (us * 1e-6) / 1e9, 1),
            "peak_gb_s": 8000.0, "frac": round(alg / (us * 1e-6) / 8e12, 4)}


def measure_masked(layer, x, steps, warmup, unmasked_ms):
    """The same workload with a padded-batch token mask (Eq. (8)): each
    sequence keeps a prefix of random length (at least half) with 5% holes.
    Mean ms per forward over `steps` back-to-back masked forwards; every
    position is still computed, `tokens_per_s` counts the unmasked ones."""
    import torch
    from scale_gla_layer_amd.synth import make_mask
    B, L, _ = x.shape
    M = make_mask(B, L, seed=2, hole_prob=0.05)
    m = torch.from_numpy(M).to(x.device)
    out = layer.new_output(B, L)
    for _ in range(warmup):
        layer.forward(x, out=out, mask=m)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, out=out, mask=m)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    return {"mask": "padded batch: random prefix lengths >= L/2, 5% holes (seed 2)",
            "token_fraction": round(float(M.mean()), 4), "us_per_step": round(ms * 1e3, 2),
            "positions_per_s": round(B * L / (ms * 1e-3), 1),
            "tokens_per_s": round(float(M.sum()) / (ms * 1e-3), 1),
            "vs_unmasked": round(unmasked_ms / ms, 4)}


def measure_norm(cfg, B, L, steps, warmup, plain_ms):
    """The same workload with the optional per-head RMS normalisation of each
    branch's output: mean ms per forward, and the normalisation pass's time
    taken as the difference to the plain forward, against the bytes it moves
    (each branch's y read and written once, plus the gains)."""
    import dataclasses
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    ncfg = dataclasses.replace(cfg, norm=True)
    X, W = make_inputs_for(ncfg, B, L)
    layer = DeviceLayer(ncfg, W)
    x = to_device(X, ncfg.dtype)
    ms, _ = time_forward(layer, x, steps, warmup, per_kernel=False)
    es = 2 if cfg.dtype == "bf16" else 4
    y_bytes = sum(B * h * (L // s) * cfg.d_v * es for s, h in zip(cfg.scales, cfg.heads))
    nbytes = 2 * y_bytes + sum(h * cfg.d_v * 4 for h in cfg.heads)
    extra_us = (ms - plain_ms) * 1e3
    return {"us_per_step": round(ms * 1e3, 2), "vs_plain": round(plain_ms / ms, 4),
            "norm_pass_us_est": round(extra_us, 2), "algorithmic_mb": round(nbytes / 1e6, 2),
            "est_gb_s": round(nbytes / (extra_us * 1e-6) / 1e9, 1) if extra_us > 0 else None,
            "peak_gb_s": 8000.0}


def make_inputs_for(cfg, B, L):
    from scale_gla_layer_amd.synth import make_inputs
    return make_inputs(cfg, B, L, seed=0)


def measure_routing(cfg, W, L=32768, steps=50, warmup=10):
    """Routing stability (Sec. 5.4, Table 3): the fusion weights of one
    L-token sequence from msgla_fusion_weights, timed over `steps` calls, and
    their mean per branch, in percent, over the first, middle and last tenth
    of the positions (n = ceil(L/10); middle window from floor((L - n)/2)).
    The weights are synthetic, so the percentages are not the printed ones."""
    import math
    import torch
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from scale_gla_layer_amd.synth import make_tokens
    layer = DeviceLayer(cfg, W)
    x = to_device(make_tokens(cfg, 1, L, seed=4), cfg.dtype)
    w = layer.fusion_weights(x)
    for _ in range(warmup):
        layer.fusion_weights(x, w_out=w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.fusion_weights(x, w_out=w)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    m = len(cfg.scales)
    wh = w[0, :, :m].double().cpu().numpy()
    n = math.ceil(L / 10)
    regions = {name: [round(float(v), 3) for v in 100.0 * wh[s0:s0 + n].mean(axis=0)]
               for name, s0 in (("first", 0), ("middle", (L - n) // 2), ("last", L - n))}
    nbytes = L * cfg.d_model * (2 if cfg.dtype == "bf16" else 4) + L * 8 * 4
    return {"seq_len": L, "us_per_call": round(us, 2), "positions_per_s": round(L / (us * 1e-6), 1),
            "hbm_gb_s": round(nbytes / (us * 1e-6) / 1e9, 1), "peak_gb_s": 8000.0,
            "percent_by_region": regions}


def measure_library_gemms(cfg, B, L, stage_ms, steps=50, warmup=10):
    """Context for the GEMM kernels: the same products as plain torch.matmul
    calls (hipBLASLt on this stack), one call per group, timed back to back.
    K1's shapes: every branch's pooled rows times its q | k | v columns, plus
    the unpooled rows times the gate first factors and fusion logits; K3's:
    every branch's y rows (coarse length) times its W_o.  Operands are
    contiguous 2-D bf16 (or fp32) tensors; only time is measured."""
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    d, dk, dv = cfg.d_model, cfg.d_k, cfg.d_v
    m = len(cfg.scales)
    rp = 16 if cfg.gate_rank <= 16 else 64
    g = torch.Generator(device="cuda").manual_seed(5)

    def mats(shapes):
        return [(torch.randn(M, K, generator=g, device="cuda", dtype=torch.float32).to(dt),
                 torch.randn(K, N, generator=g, device="cuda", dtype=torch.float32).to(dt))
                for M, K, N in shapes]

    k1 = [(B * (L // s), d, h * (2 * dk + dv)) for s, h in zip(cfg.scales, cfg.heads)]
    k1.append((B * L, d, m * rp + (16 if m > 1 else 0)))
    k3 = [(B * (L // s), h * dv, d) for s, h in zip(cfg.scales, cfg.heads)]
    out = {}
    for name, shapes in (("k1", k1), ("k3", k3)):
        ops = mats(shapes)
        for _ in range(warmup):
            for a, w in ops:
                torch.matmul(a, w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            for a, w in ops:
                torch.matmul(a, w)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        fl = sum(2.0 * M * K * N for M, K, N in shapes)
        out[name] = {"shapes": [list(t) for t in shapes], "library_us": round(us, 2),
                     "library_tflops": round(fl / (us * 1e-6) / 1e12, 1)}
        del ops
    out["k1"]["ours_us"] = round(stage_ms.get("proj", 0.0) * 1e3, 2)
    out["k3"]["ours_us"] = round((stage_ms.get("out_coarse", 0.0) + stage_ms.get("hold_fuse", 0.0)) * 1e3, 2)
    out["note"] = ("ours: K1 (one launch, with its q/k/v/gate/fusion epilogues) and K3c + K3f "
                   "(with the hold and fusion epilogue) from the event pass; library: the bare "
                   "products, one torch.matmul per group")
    return out


def measure_training(workload="main", steps=20, warmup=5):
    """One training step of the layer on one input, each part timed with events over
    `steps` back-to-back calls after clock settling (dO a seeded N(0, 1) tensor):
    the step is msgla_forward_train + msgla_backward_saved (the backward reads the
    intermediates the training forward kept); msgla_forward + msgla_backward (which
    recomputes them) is reported beside it.  The backward's algorithmic flops are
    taken as twice the forward's (each product of the forward appears twice in the
    backward: once for the input's gradient, once for the weight's)."""
    import numpy as np
    import torch
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from scale_gla_layer_amd.synth import make_inputs, round_to
    wl = WORKLOADS[workload]
    cfg, B, L = wl.cfg, wl.batch, wl.seq_len
    X, W = make_inputs(cfg, B, L, seed=0, gate_bias=wl.gate_bias)
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    dO = to_device(round_to(np.random.default_rng(1).normal(0.0, 1.0, X.shape), cfg.dtype), cfg.dtype)
    settle_clocks(layer, x, max_s=1.0)
    out = layer.new_output(B, L)
    dx, grads = layer.backward(x, dO)
    fwd_t = lambda: layer.forward_train(x, out=out)
    bwd_s = lambda: layer.backward(x, dO, dx=dx, grads=grads, saved=True)
    for _ in range(warmup):
        layer.forward(x, out=out)
        layer.backward(x, dO, dx=dx, grads=grads)
        fwd_t()
        bwd_s()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    fwd = timed(lambda: layer.forward(x, out=out))
    fwdt = timed(fwd_t)
    bwd = timed(bwd_s)
    bwd_r = timed(lambda: layer.backward(x, dO, dx=dx, grads=grads))
    step = timed(lambda: (fwd_t(), bwd_s()))
    step_r = timed(lambda: (layer.forward(x, out=out), layer.backward(x, dO, dx=dx, grads=grads)))
    alg = algorithmic(cfg, B, L)
    peak = PEAK["bf16_mfma_tflops"] if cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
    bwd_flops = 2 * alg["flops"]
    del layer, x, dO, out, dx, grads
    return {"workload": workload, "batch": B, "seq_len": L, "forward_us": round(fwd, 1),
            "forward_train_us": round(fwdt, 1), "backward_us": round(bwd, 1),
            "backward_recompute_us": round(bwd_r, 1), "step_us": round(step, 1),
            "step_recompute_us": round(step_r, 1),
            "tokens_per_s": round(B * L / (step * 1e-6), 1),
            "tokens_per_s_recompute": round(B * L / (step_r * 1e-6), 1),
            "backward_algorithmic_gflop": round(bwd_flops / 1e9, 2),
            "backward_tflops": round(bwd_flops / (bwd * 1e-6) / 1e12, 1),
            "backward_roofline_frac": round(bwd_flops / (peak * 1e12) / (bwd * 1e-6), 4)}


def device_info():
    """What the line was measured on: the GPU's name, gfx architecture and
    CU count, the HIP runtime torch was built against, and the host CPU."""
    import torch
    props = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count,
            "memory_gib": round(props.total_memory / 2**30, 1),
            "hip": torch.version.hip, "torch": torch.__version__, "host_cpu": cpu,
            "host_cores": len(os.sched_getaffinity(0))}


def settle_clocks(layer, x, batch=20, tol=0.01, max_s=3.0):
    """Runs forwards in batches of `batch` until the mean time of a batch is
    within `tol` of the previous one (the shader clock settles under load;
    the first forwards after a pause run a few percent slow), at most max_s
    seconds.  Independent of --warmup.  Returns what it took."""
    import torch
    B, L, _ = x.shape
    out = layer.new_output(B, L)
    t_start = time.perf_counter()
    prev, n, means = None, 0, []
    while True:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(batch):
            layer.forward(x, out=out)
        torch.cuda.synchronize()
        mean = (time.perf_counter() - t0) / batch
        n += batch
        means.append(mean)
        if prev is not None and abs(mean - prev) <= tol * prev:
            break
        if time.perf_counter() - t_start >= max_s:
            break
        prev = mean
    return {"forwards": n, "seconds": round(time.perf_counter() - t_start, 3),
            "last_batch_us": round(means[-1] * 1e6, 2),
            "first_batch_us": round(means[0] * 1e6, 2)}


def time_forward(layer, x, steps, warmup, per_kernel=True):
    """Mean ms per forward over `steps` back-to-back forwards (no events inside
    the forwards), then, if per_kernel, mean ms per kernel from a second pass
    of `steps` forwards with the library's stage events (each event marker adds
    a few microseconds between kernels, so that pass is not the headline)."""
    import torch
    B, L, _ = x.shape
    out = layer.new_output(B, L)
    for _ in range(warmup):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stage_ms = {}
    if per_kernel:
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in STAGES] for _ in range(steps)]
        for row in ev:  # materialise the HIP events before handing them to the library
            for a, b in row:
                a.record()
                b.record()
        torch.cuda.synchronize()
        for k in range(steps):
            layer.forward(x, out=out, events=([a for a, _ in ev[k]], [b for _, b in ev[k]]))
        torch.cuda.synchronize()
        stage_ms = {name: float(np.mean([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)]))
                    for i, name in enumerate(STAGES)}
    return dt / steps * 1e3, stage_ms


def per_call_distribution(layer, x, calls=100, scrub=False):
    """p10 / p50 / p90 of `calls` forwards, each bracketed by its own pair of
    events.  scrub=True writes a 512 MiB buffer before every call, which evicts
    the 256 MB MALL, so each forward starts with cold caches (its inputs and
    weights come from HBM)."""
    import torch
    B, L, _ = x.shape
    out = layer.new_output(B, L)
    junk = torch.empty(512 << 20, dtype=torch.uint8, device=x.device) if scrub else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for _ in range(5):
        layer.forward(x, out=out)
    for a, b in ev:
        if junk is not None:
            junk.zero_()
        a.record()
        layer.forward(x, out=out)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"calls": calls, "p10": round(float(np.percentile(t, 10)), 2),
            "p50": round(float(np.percentile(t, 50)), 2), "p90": round(float(np.percentile(t, 90)), 2)}


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(kernel):
        log(f"[bench] {path}: counters predate the current {kernel} sources; traffic = null")
        return None
    return rec.get("hbm_bytes_per_dispatch")


def cpu_worker(workload: str, first: int, stride: int, min_s: float):
    """One single-threaded worker of the CPU baseline: the oracle on sequences
    first, first + stride, ... of the workload's seeded batch (cycling) until
    min_s seconds of oracle work; prints {"tokens", "seconds"}."""
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.synth import make_inputs
    wl = WORKLOADS[workload]
    X, W = make_inputs(wl.cfg, wl.batch, wl.seq_len, seed=0, gate_bias=wl.gate_bias)
    B, L, _ = X.shape
    done, k, t0 = 0, first, time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        b = k % B
        orc.layer_forward(X[b: b + 1], W, wl.cfg)
        done += L
        k += stride
    print(json.dumps({"tokens": done, "seconds": time.perf_counter() - t0}), flush=True)


def cpu_decode_baseline(workload: str = "sweep_1248", steps: int = 64):
    """The oracle's streaming step on the host (part of the CPU baseline leg):
    the decode workload's batch from an empty cache (a step's cost does not
    depend on the position), `steps` steps in one process."""
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.synth import make_inputs
    wl = WORKLOADS[workload]
    X, W = make_inputs(wl.cfg, wl.batch, steps, seed=0)
    st = orc.init_state(wl.cfg, wl.batch)
    t0 = time.perf_counter()
    for t in range(steps):
        _, st = orc.decode_step(st, X[:, t], W, wl.cfg)
    us = (time.perf_counter() - t0) / steps * 1e6
    return {"workload": workload, "batch": wl.batch, "steps": steps, "us_per_step": round(us, 1),
            "tokens_per_s": round(wl.batch / (us * 1e-6), 1)}


def cpu_training_baseline(workload: str = "main"):
    """The oracle's forward and backward (its vector-Jacobian product) of one
    sequence of the workload in one process (part of the CPU baseline leg)."""
    import numpy as np
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.synth import make_inputs
    wl = WORKLOADS[workload]
    X, W = make_inputs(wl.cfg, 1, wl.seq_len, seed=0)
    dO = np.random.default_rng(1).normal(0.0, 1.0, X.shape)
    t0 = time.perf_counter()
    orc.layer_forward(X, W, wl.cfg)
    orc.layer_backward(X, W, wl.cfg, dO)
    s = time.perf_counter() - t0
    return {"workload": workload, "sample": f"one sequence of {wl.seq_len} tokens, forward + backward, "
            "one process", "seconds": round(s, 2), "tokens_per_s": round(wl.seq_len / s, 1)}


def cpu_baseline(workload: str, min_s: float = 10.0):
    """The oracle as it stands, on the host's cores: one single-threaded
    process per core (BLAS limited to one thread), each cycling over the
    workload's sequences until min_s seconds of work; tokens/s = all tokens
    over the longest worker's oracle time (input generation excluded)."""
    import subprocess
    from scale_gla_layer_amd.config import WORKLOADS
    L = WORKLOADS[workload].seq_len
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               BLIS_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker",
                               workload, str(i), str(cores), str(min_s)],
                              stdout=subprocess.PIPE, env=env, text=True) for i in range(cores)]
    res = []
    for p in procs:
        outp, _ = p.communicate(timeout=600)
        if p.returncode != 0:
            raise RuntimeError(f"CPU baseline worker failed ({p.returncode})")
        res.append(json.loads(outp.strip().splitlines()[-1]))
    tokens = sum(r["tokens"] for r in res)
    secs = max(r["seconds"] for r in res)
    model = ""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": tokens / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{tokens // L} sequence forwards of {L} tokens of the {workload} "
                      f"workload over {cores} single-threaded processes ({secs:.1f} s each; fp64 "
                      f"NumPy, token-by-token recurrence; {model})"}


PROFILE_COMMANDS = {
    "ktrace": "rocprofv3 --kernel-trace --stats -f csv -d {d}/ktrace -o main -- "
              "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-gla --no-per-call --no-decode --no-mask --no-routing --no-norm --no-workloads --no-library-gemms --no-training",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d {d}/pmc_fetch -o main -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-gla --no-per-call --no-decode --no-mask --no-routing --no-norm --no-workloads --no-library-gemms --no-training",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d {d}/pmc_write -o main -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-gla --no-per-call --no-decode --no-mask --no-routing --no-norm --no-workloads --no-library-gemms --no-training",
    "util": "rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LDSBankConflict MfmaFlopsBF16 MfmaFlopsF32 "
            "-f csv -d {d}/pmc_util -o main -- "
            "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-gla --no-per-call --no-decode --no-mask --no-routing --no-norm --no-workloads --no-library-gemms --no-training",
    "cal_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d {d}/cal_fetch -o copy -- "
                 "python3 bench.py --copy-calibration",
    "cal_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d {d}/cal_write -o copy -- "
                 "python3 bench.py --copy-calibration",
    "dec_ktrace": "rocprofv3 --kernel-trace --stats -f csv -d {d}/dec_ktrace -o decode -- "
                  "python3 bench.py --only-decode",
    "bwd_ktrace": "rocprofv3 --kernel-trace --stats -f csv -d {d}/bwd_ktrace -o backward -- "
                  "python3 bench.py --only-training --no-gla",
}


def _short(name: str) -> str:
    for k in KERNELS.values():
        if k in name:
            return k
    return name[:48]


def _counter_means(path: str) -> dict:
    import csv
    acc = {}
    with open(path, newline="", encoding="utf-8") as f:
        for r in csv.DictReader(f):
            acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_training_profile(d, workload, wl, cmds, out_dir):
    """profiles/kernels_training_<workload>.md from the bwd_ktrace run, if present."""
    import csv
    # the training step: the training forward, the backward from its saved intermediates,
    # and the recomputing backward
    bwd_csv = os.path.join(d, "bwd_ktrace", "backward_kernel_stats.csv")
    if os.path.exists(bwd_csv):
        with open(bwd_csv, newline="", encoding="utf-8") as f:
            bstats = list(csv.DictReader(f))
        brows = [f"# Kernel trace, training step (forward + backward), workload {workload} "
                 f"({wl.description})", "",
                 "Command (from the repository root, `<out>` any output directory):", "",
                 f"    {cmds['bwd_ktrace']}", "",
                 "Clock settling forwards, then 5 warm-up rounds and 20 calls each of the forward, "
                 "the training forward (msgla_forward_train), the backward from its saved "
                 "intermediates (msgla_backward_saved), the recomputing backward (msgla_backward), "
                 "and the two steps (training forward + saved backward; forward + recomputing "
                 "backward). The recomputing backward runs the forward's kernels except the fused "
                 "output launch, so those appear more often than k3f_fine_fuse. rocBLAS kernels are "
                 "named by their macro tile; k_bwd_walk runs once per direction (states, state "
                 "gradients) per backward.", "",
                 "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
        import re
        for r in bstats:
            name = r["Name"]
            if name.startswith("Cijk"):
                mt = re.search(r"MT\d+x\d+x\d+", name)
                short = "rocBLAS " + (mt.group(0) if mt else "gemm") + (" fp32" if "_SB_" in name else "")
            else:
                short = _short(name)
                m = re.search(r"(k_bwd_[A-Za-z0-9_]*?)(?=I[DfL]|E|<|\(|$)", name)
                if m:
                    short = m.group(1)
                    if short in ("k_bwd_outer", "k_bwd_outer_split"):
                        short += " (dS)" if ("Lb1E" in name or "true>" in name) else " (S)"
                    if short == "k_bwd_walk":
                        short += " (dS)" if ("Lb1E" in name or ", true," in name) else " (S)"
                if "k_bwd_gemm" in name:
                    # storage-type output: the pooled inputs' gradient; fp32: dLoss/do
                    short = "k_bwd_gemm " + ("(dxp)" if ("DF16bDF16b" in name or "IffE" in name) else "(do)")
            brows.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
        with open(os.path.join(out_dir, f"kernels_training_{workload}.md"), "w", encoding="utf-8") as f:
            f.write("\n".join(brows) + "\n")


def summarize_profiles(d: str, workload: str = "main"):
    """Writes profiles/kernels_<workload>.md (kernel trace) and, per kernel of
    the forward, profiles/<kernel>_<workload>_traffic.json (FETCH_SIZE and
    WRITE_SIZE per dispatch scaled by the plain-copy calibration) from the
    rocprofv3 output directories under d (see PROFILE_COMMANDS)."""
    import csv
    from scale_gla_layer_amd.config import WORKLOADS
    wl = WORKLOADS[workload]
    alg = algorithmic(wl.cfg, wl.batch, wl.seq_len)["stage"]
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    cmds = {k: v.format(d="<out>") for k, v in PROFILE_COMMANDS.items()}

    if not os.path.exists(os.path.join(d, "ktrace", "main_kernel_stats.csv")):
        summarize_training_profile(d, workload, wl, cmds, out_dir)
        return
    with open(os.path.join(d, "ktrace", "main_kernel_stats.csv"), newline="", encoding="utf-8") as f:
        stats = list(csv.DictReader(f))
    lines = [f"# Kernel trace, workload {workload} ({wl.description})", "",
             "Command (from the repository root, `<out>` any output directory):", "",
             f"    {cmds['ktrace']}", "",
             "The forwards of one short run under the tracer: clock settling (batches of 20 "
             "until two agree within 1%), 5 warm-up, 20 timed and 20 with stage events.", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(os.path.join(out_dir, f"kernels_{workload}.md"), "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")

    cal_f = _counter_means(os.path.join(d, "cal_fetch", "copy_counter_collection.csv"))
    cal_w = _counter_means(os.path.join(d, "cal_write", "copy_counter_collection.csv"))
    # the copy is the runtime's buffer-copy blit of COPY_CAL_BYTES (read once, written once)
    ref_f = cal_f["__amd_rocclr_copyBuffer"][0] * 1024.0
    ref_w = cal_w["__amd_rocclr_copyBuffer"][0] * 1024.0
    f_fac, w_fac = COPY_CAL_BYTES / ref_f, COPY_CAL_BYTES / ref_w
    fetch = _counter_means(os.path.join(d, "pmc_fetch", "main_counter_collection.csv"))
    write = _counter_means(os.path.join(d, "pmc_write", "main_counter_collection.csv"))
    # the kernels' source hashes as the counted runs printed them (their logs,
    # <d>/fetch.log and <d>/write.log): a record is only as current as the code
    # it was counted on
    run_hashes = {}
    for name in ("fetch", "write"):
        try:
            with open(os.path.join(d, f"{name}.log"), encoding="utf-8") as f:
                for ln in f:
                    if "[bench] kernel source hashes:" in ln:
                        h = json.loads(ln.split("kernel source hashes:", 1)[1])
                        run_hashes = h if name == "fetch" else (run_hashes if run_hashes == h else {})
        except OSError:
            run_hashes = {}
            break
    rows = ["# HBM traffic per dispatch, workload " + workload, "",
            "Commands (from the repository root):", ""] + [f"    {cmds[k]}" for k in
                                                        ("fetch", "write", "cal_fetch", "cal_write")]
    rows += ["", f"Calibration: a plain copy of {COPY_CAL_BYTES} bytes reads FETCH_SIZE "
             f"{ref_f / 1024:.0f} KiB and WRITE_SIZE {ref_w / 1024:.0f} KiB, so bytes = "
             f"FETCH_SIZE x 1024 x {f_fac:.3f} + WRITE_SIZE x 1024 x {w_fac:.3f}.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB | algorithmic | traffic / algorithmic |",
             "|---|---|---|---|---|---|"]
    for stage, kernel in KERNELS.items():
        if kernel not in fetch or kernel not in write:
            continue
        fk, wk = fetch[kernel][0], write[kernel][0]
        hbm = fk * 1024 * f_fac + wk * 1024 * w_fac
        bound, amount = alg[stage]
        alg_txt = f"{amount / 1e6:.1f} MB" if bound == "hbm" else f"{amount / 1e9:.1f} GFLOP"
        ratio = f"{hbm / amount:.2f}" if bound == "hbm" and amount else "-"
        rows.append(f"| {kernel} | {fk:.0f} | {wk:.0f} | {hbm / 1e6:.1f} | {alg_txt} | {ratio} |")
        rec = {"kernel": kernel, "workload": workload, "source_hash": run_hashes.get(kernel, "unknown"),
               "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
               "fetch_factor": f_fac, "write_factor": w_fac, "hbm_bytes_per_dispatch": round(hbm),
               "dispatches": fetch[kernel][1], "commands": [cmds[k] for k in
                                                            ("fetch", "write", "cal_fetch", "cal_write")]}
        with open(os.path.join(out_dir, f"{kernel}_{workload}_traffic.json"), "w", encoding="utf-8") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    with open(os.path.join(out_dir, f"traffic_{workload}.md"), "w", encoding="utf-8") as f:
        f.write("\n".join(rows) + "\n")

    # utilisation counters (derived metrics of rocprofv3), next to the trace's
    # average durations and the traffic above
    util_csv = os.path.join(d, "pmc_util", "main_counter_collection.csv")
    if os.path.exists(util_csv):
        per = {}
        with open(util_csv, newline="", encoding="utf-8") as f:
            for r in csv.DictReader(f):
                per.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
        avg_us = {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
        urows = [f"# Utilisation counters per dispatch, workload {workload}", "",
                 "Command (from the repository root):", "", f"    {cmds['util']}", "",
                 "MfmaUtil: MFMA-busy cycles over (GPU-active cycles x SIMDs); VALUBusy: "
                 "cycles with a VALU instruction (MFMA included) active per CU; LdsUtil: "
                 "cycles the LDS is indexed per CU; LDSBankConflict: bank-conflict cycles per "
                 "CU, all in percent of the kernel's active cycles. MFMA TFLOP/s and HBM GB/s "
                 "divide the counted MFMA flops and the calibrated traffic "
                 f"(traffic_{workload}.md) by the trace's average duration "
                 f"(kernels_{workload}.md); peaks 2500 TFLOP/s (bf16 dense), 157.3 (fp32) and "
                 "8000 GB/s.", "",
                 "| kernel | avg us | MfmaUtil % | VALUBusy % | LdsUtil % | LDS conflict % | "
                 "MFMA GFLOP | MFMA TFLOP/s | HBM MB | HBM GB/s |",
                 "|---|---|---|---|---|---|---|---|---|---|"]
        for stage, kernel in KERNELS.items():
            if kernel not in per or kernel not in avg_us:
                continue
            m = {k: sum(v) / len(v) for k, v in per[kernel].items()}
            us = avg_us[kernel]
            fl = m.get("MfmaFlopsBF16", 0.0) + m.get("MfmaFlopsF32", 0.0)
            hbm = None
            if kernel in fetch and kernel in write:
                hbm = fetch[kernel][0] * 1024 * f_fac + write[kernel][0] * 1024 * w_fac
            urows.append(
                f"| {kernel} | {us:.2f} | {m.get('MfmaUtil', 0):.1f} | {m.get('VALUBusy', 0):.1f} | "
                f"{m.get('LdsUtil', 0):.1f} | {m.get('LDSBankConflict', 0):.2f} | {fl / 1e9:.2f} | "
                f"{fl / (us * 1e-6) / 1e12:.0f} | "
                + (f"{hbm / 1e6:.1f} | {hbm / (us * 1e-6) / 1e9:.0f} |" if hbm is not None else "- | - |"))
        with open(os.path.join(out_dir, f"counters_{workload}.md"), "w", encoding="utf-8") as f:
            f.write("\n".join(urows) + "\n")
    # the streaming decode step (prefill, then the timed eager steps and the
    # graph replays of measure_decode)
    dec_csv = os.path.join(d, "dec_ktrace", "decode_kernel_stats.csv")
    if os.path.exists(dec_csv):
        with open(dec_csv, newline="", encoding="utf-8") as f:
            dstats = list(csv.DictReader(f))
        dwl = WORKLOADS["sweep_1248"]
        drows = [f"# Kernel trace, decode step, workload sweep_1248 ({dwl.description})", "",
                 "Command (from the repository root, `<out>` any output directory):", "",
                 f"    {cmds['dec_ktrace']}", "",
                 "Two prefills of 4096 tokens (the forward's kernels), then 288 eager decode "
                 "steps and 288 graph replays, B = 16; each step is k_dec_proj, k_dec_state "
                 "and k_dec_out.", "",
                 "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
        for r in dstats:
            name = r["Name"]
            short = next((k for k in ("k_dec_proj", "k_dec_state", "k_dec_out") if k in name), _short(name))
            drows.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
        with open(os.path.join(out_dir, "kernels_decode_sweep_1248.md"), "w", encoding="utf-8") as f:
            f.write("\n".join(drows) + "\n")
    summarize_training_profile(d, workload, wl, cmds, out_dir)
    log(f"[bench] wrote profiles for {workload} from {d}")


def copy_calibration():
    """A plain device copy of COPY_CAL_BYTES (read once, written once), 5 times."""
    import torch
    src = torch.ones(COPY_CAL_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 copies of {COPY_CAL_BYTES} bytes")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gla", action="store_true", help="skip the single-scale GLA comparison")
    ap.add_argument("--no-decode", action="store_true", help="skip the streaming decode timing")
    ap.add_argument("--no-mask", action="store_true", help="skip the masked-forward timing")
    ap.add_argument("--no-routing", action="store_true", help="skip the routing-stability timing")
    ap.add_argument("--no-norm", action="store_true", help="skip the normalised-forward timing")
    ap.add_argument("--no-per-call", action="store_true",
                    help="skip the per-call (warm and cold-MALL) distributions")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain-copy reference kernel for counter scaling")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output under DIR (no GPU)")
    ap.add_argument("--no-library-gemms", action="store_true",
                    help="skip timing the GEMM shapes as plain library calls")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' forward lines (GLA, long, sweeps)")
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the streaming decode step and print its JSON")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the training-step (forward + backward) timing")
    ap.add_argument("--only-training", action="store_true",
                    help="time only the training step (main and GLA baseline) and print its JSON")
    ap.add_argument("--cpu-worker", nargs=4, metavar=("WORKLOAD", "FIRST", "STRIDE", "SECONDS"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_worker:
        w, first, stride, secs = args.cpu_worker
        cpu_worker(w, int(first), int(stride), float(secs))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this layer's path is built and timed on a single "
              f"MI355X); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.only_training:
        tr = measure_training(args.workload)
        if not args.no_gla and args.workload != "gla_baseline":
            tr["gla"] = measure_training("gla_baseline")
            tr["ratio_vs_gla"] = round(tr["tokens_per_s"] / tr["gla"]["tokens_per_s"], 4)
        print(json.dumps(tr), flush=True)
        return
    if args.only_decode:
        dec = measure_decode()
        log(f"[bench] decode {dec['workload']} B={dec['batch']}: {dec['us_per_step']} us/step")
        print(json.dumps(dec), flush=True)
        return

    import torch  # noqa: F401
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from scale_gla_layer_amd.synth import make_inputs

    wl = WORKLOADS[args.workload]
    cfg, B, L = wl.cfg, wl.batch, wl.seq_len
    log(f"[bench] workload {wl.name}: {wl.description}")
    log("[bench] kernel source hashes: " + json.dumps({k: kernel_source_hash(k) for k in KERNEL_SOURCES}))
    X, W = make_inputs(cfg, B, L, seed=0, gate_bias=wl.gate_bias)
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    settle = settle_clocks(layer, x)
    log(f"[bench] clocks settled after {settle['forwards']} forwards ({settle['seconds']} s): "
        f"{settle['first_batch_us']} -> {settle['last_batch_us']} us")
    ms, stage_ms = time_forward(layer, x, args.steps, args.warmup)
    tok_s = B * L / (ms * 1e-3)
    log(f"[bench] {ms * 1e3:.1f} us/step, {tok_s / 1e6:.1f} M tokens/s; kernels (us, event pass): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in stage_ms.items()))

    warm = cold = None
    if not args.no_per_call:
        warm = per_call_distribution(layer, x)
        cold = per_call_distribution(layer, x, scrub=True)
        log(f"[bench] per call (us): warm p10/p50/p90 {warm['p10']}/{warm['p50']}/{warm['p90']}, "
            f"cold MALL {cold['p10']}/{cold['p50']}/{cold['p90']}")

    alg = algorithmic(cfg, B, L)
    peak_f = PEAK["bf16_mfma_tflops"] if cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
    layer_tflops = alg["flops"] / (ms * 1e-3) / 1e12
    t_roof = max(alg["flops"] / (peak_f * 1e12), alg["bytes"] / (PEAK["hbm_gbs"] * 1e9))
    stages = {}
    for name, t in stage_ms.items():
        b, a = alg["stage"][name]
        if a <= 0:
            continue
        rate = a / (t * 1e-3) / (1e12 if b == "mfma" else 1e9)
        peak = peak_f if b == "mfma" else PEAK["hbm_gbs"]
        stages[name] = {"kernel": KERNELS[name], "us": round(t * 1e3, 2), "bound": b,
                        "achieved": round(rate, 1), "unit": "TFLOP/s" if b == "mfma" else "GB/s",
                        "peak": peak, "frac": round(rate / peak, 4),
                        "algorithmic": a}
    dom = max(stages, key=lambda k: stages[k]["us"])
    d = stages[dom]
    roofline = {"bound": d["bound"], "kernel": d["kernel"], "achieved": d["achieved"],
                "peak": d["peak"], "unit": d["unit"], "frac": d["frac"],
                "traffic": traffic_from_profile(d["kernel"], wl.name),
                "algorithmic_per_launch": d["algorithmic"]}

    libg = None
    if not args.no_library_gemms and stage_ms:
        libg = measure_library_gemms(cfg, B, L, stage_ms)
        log(f"[bench] library GEMMs of the same shapes: K1's {libg['k1']['library_us']} us "
            f"({libg['k1']['library_tflops']} TFLOP/s) against K1 {libg['k1']['ours_us']} us; "
            f"K3's {libg['k3']['library_us']} us against K3c + K3f {libg['k3']['ours_us']} us")

    masked = None
    if not args.no_mask:
        masked = measure_masked(layer, x, args.steps, args.warmup, ms)
        log(f"[bench] masked forward {masked['us_per_step']} us/step ({masked['vs_unmasked']:.3f} of the "
            f"unmasked rate), {masked['token_fraction']:.3f} of the positions are tokens")

    normed = None
    if not args.no_norm:
        normed = measure_norm(cfg, B, L, args.steps, args.warmup, ms)
        log(f"[bench] normalised forward {normed['us_per_step']} us/step; normalisation pass about "
            f"{normed['norm_pass_us_est']} us for {normed['algorithmic_mb']} MB")

    routing = None
    if not args.no_routing and len(cfg.scales) > 1:
        routing = measure_routing(cfg, W)
        log(f"[bench] routing: fusion weights of a {routing['seq_len']}-token sequence in "
            f"{routing['us_per_call']} us ({routing['hbm_gb_s']} GB/s); percent by region "
            f"{routing['percent_by_region']}")

    def workload_line(name, steps):
        """Another workload's forward, timed like the headline: tokens/s and the
        layer roofline fraction."""
        owl = WORKLOADS[name]
        Xo, Wo = make_inputs(owl.cfg, owl.batch, owl.seq_len, seed=0, gate_bias=owl.gate_bias)
        olayer = DeviceLayer(owl.cfg, Wo)
        xo = to_device(Xo, owl.cfg.dtype)
        settle_clocks(olayer, xo, max_s=1.0)
        oms, _ = time_forward(olayer, xo, steps, max(5, steps // 4), per_kernel=False)
        oalg = algorithmic(owl.cfg, owl.batch, owl.seq_len)
        opeak = PEAK["bf16_mfma_tflops"] if owl.cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
        oroof = max(oalg["flops"] / (opeak * 1e12), oalg["bytes"] / (PEAK["hbm_gbs"] * 1e9))
        del olayer, xo
        return {"batch": owl.batch, "seq_len": owl.seq_len, "scales": list(owl.cfg.scales),
                "heads": list(owl.cfg.heads), "us_per_step": round(oms * 1e3, 2),
                "tokens_per_s": round(owl.batch * owl.seq_len / (oms * 1e-3), 1),
                "algorithmic_gflop": round(oalg["flops"] / 1e9, 2),
                "t_roof_us": round(oroof * 1e6, 2), "layer_roofline_frac": round(oroof / (oms * 1e-3), 4)}

    ratio_vs_gla = None
    gla = None
    others = {}
    if not args.no_gla and args.workload != "gla_baseline":
        others["gla_baseline"] = workload_line("gla_baseline", args.steps)
        gla = others["gla_baseline"]["tokens_per_s"]
        ratio_vs_gla = tok_s / gla
        log(f"[bench] GLA baseline {others['gla_baseline']['us_per_step']} us/step, {gla / 1e6:.1f} M "
            f"tokens/s ({others['gla_baseline']['layer_roofline_frac']} of its roofline); "
            f"ratio {ratio_vs_gla:.3f}")
    if not args.no_workloads:
        for name in ("long", "sweep_1248", "sweep_24"):
            if name == args.workload:
                continue
            others[name] = workload_line(name, min(args.steps, 100))
            o = others[name]
            log(f"[bench] {name}: {o['us_per_step']} us/step, {o['tokens_per_s'] / 1e6:.1f} M tokens/s, "
                f"{o['layer_roofline_frac']} of its layer roofline ({o['t_roof_us']} us)")

    dec = None
    if not args.no_decode:
        dec = measure_decode()
        log(f"[bench] decode {dec['workload']} B={dec['batch']}: {dec['us_per_step']} us/step "
            f"({dec['us_per_step_graph']} from a captured graph), "
            f"{dec['achieved_gb_s']} GB/s ({dec['algorithmic_mb_per_step']} MB/step), host "
            f"{dec['host_us_per_call']} us/call")

    training = None
    if not args.no_training:
        training = measure_training(wl.name)
        log(f"[bench] training step {training['step_us']} us ({training['forward_train_us']} training "
            f"forward + {training['backward_us']} backward from the saved intermediates), "
            f"{training['tokens_per_s'] / 1e6:.2f} M tokens/s; with the recomputing backward "
            f"{training['step_recompute_us']} us ({training['forward_us']} + "
            f"{training['backward_recompute_us']})")
        if args.workload != "gla_baseline" and not args.no_gla:
            training["gla"] = measure_training("gla_baseline")
            training["ratio_vs_gla"] = round(training["tokens_per_s"] / training["gla"]["tokens_per_s"], 4)
            log(f"[bench] GLA baseline training step {training['gla']['step_us']} us; MS-GLA / GLA "
                f"training throughput {training['ratio_vs_gla']}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on the host ...")
        cpu = cpu_baseline(wl.name)
        log(f"[bench] oracle {cpu['value']:.0f} tokens/s ({cpu['sample']})")
        if training is not None:
            cpu["training"] = cpu_training_baseline(wl.name)
            log(f"[bench] oracle forward + backward {cpu['training']['tokens_per_s']} tokens/s "
                f"({cpu['training']['sample']})")
        if dec is not None:
            cpu["decode"] = cpu_decode_baseline(dec["workload"])
            log(f"[bench] oracle decode step {cpu['decode']['us_per_step']} us (B={cpu['decode']['batch']}, "
                f"one process)")

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
        "roofline": roofline,
        "layer_roofline": {"algorithmic_gflop": round(alg["flops"] / 1e9, 2),
                           "algorithmic_mb": round(alg["bytes"] / 1e6, 2),
                           "achieved_tflops": round(layer_tflops, 1),
                           "t_roof_us": round(t_roof * 1e6, 2),
                           "frac": round(t_roof / (ms * 1e-3), 4)},
        "kernels": stages,
        "library_gemms": libg,
        "device": device_info(),
        "settle": settle,
        "per_call_us": warm,
        "per_call_cold_mall_us": cold,
        "cold_mall_tokens_per_s": None if cold is None else round(B * L / (cold["p50"] * 1e-6), 1),
        "workloads": others,
        "ratio_vs_gla": None if ratio_vs_gla is None else round(ratio_vs_gla, 4),
        "gla_tokens_per_s": None if gla is None else round(gla, 1),
        "decode": dec,
        "training": training,
        "masked": masked,
        "routing": routing,
        "norm": normed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
