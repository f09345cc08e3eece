"""Benchmark: one MoE layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer (routing metadata, permute, grouped
SwiGLU GEMMs, combine, and every backward step) over one batch of seeded
synthetic input already resident in HBM. The default workload is the large
expert pool: T = 16384 tokens, d_model = 2048, 128 experts, top-4, d_ff = 1024,
bf16, uniform random routing with Dirichlet(1) gate weights (the pages'
headline system benchmarks are random-routed). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_MXFP8_TFLOPS = 5033.2   # MI355X dense fp8 / MXFP8 MFMA

METRIC = "MoE layer fwd+bwd tokens/s at E=128 top-4 d=2048; grouped-GEMM % MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(name, wl, n_rows, R):
    """(kind, algorithmic amount per launch): flops for GEMMs, bytes otherwise."""
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    rows = n_rows
    gemm = {"gg_fwd_gate_up": 4, "gg_fwd_down": 2, "gg_dgrad_down": 2, "gg_wgrad_down": 2,
            "gg_dgrad_gate_up": 4, "gg_wgrad_gate_up": 4}
    if name in gemm:
        return "mfma", gemm[name] * rows * d * F
    b = {
        "permute": T * d * 2 + rows * d * 2 + R * 4,
        "combine": R * d * 2 + T * d * 2 + R * 8,
        "combine_bwd": T * d * 2 + 2 * R * d * 2 + R * 12,
        "permute_bwd": R * d * 2 + T * d * 2 + R * 4,
        "offsets": R * 4 * 3 + rows * 4,
        "router_gemm": T * d * 2 + T * E * 4,
        "route": T * E * 4 + T * k * 8,
        "route_bwd": T * k * 12 + T * E * 4,
        "router_gemm_bwd": T * d * 2 + T * E * 4 + d * E * 2,
    }
    return "hbm", b[name]


def stage_algorithmic_bytes(name, wl, n_rows, R):
    """Bytes a stage must move at least once (inputs read, outputs written)."""
    d, F = wl.d, wl.F
    W = wl.E * d * F * 2            # one bf16 expert weight tensor, all experts
    x, f = n_rows * d * 2, n_rows * F * 2
    gemm = {"gg_fwd_gate_up": x + 2 * W + 3 * f, "gg_fwd_down": f + W + x,
            "gg_dgrad_down": x + W + 4 * f, "gg_dgrad_gate_up": 2 * f + 2 * W + x,
            "gg_wgrad_down": f + x + W, "gg_wgrad_gate_up": x + 2 * f + 2 * W}
    if name in gemm:
        return gemm[name]
    return stage_work(name, wl, n_rows, R)[1]


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "routing_grouped_expert_router_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources; else None."""
    from profile_summary import read_traffic_table
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    try:
        tab = read_traffic_table(path)
    except ValueError:
        return None
    ent = tab.get(workload, {}).get(stage)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(wl, inp, budget_s):
    """The oracle, as it stands, on the first T_s tokens of the same workload
    (all experts, full weights), doubling T_s until one fwd+bwd takes at least
    budget_s seconds of wall time."""
    import numpy as np
    import oracle.moe as om
    from oracle.numerics import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    p = {n: bf16_bits_to_f64(inp[n]) for n in ("w_gate", "w_up", "w_down")}
    Ts = 1024
    while True:
        q = dict(p)
        q["x"] = bf16_bits_to_f64(inp["x"][:Ts])
        dy = bf16_bits_to_f64(inp["dy"][:Ts])
        if "topk_idx" in inp:
            q["topk_idx"], q["topk_w"] = inp["topk_idx"][:Ts], inp["topk_w"][:Ts].astype(np.float64)
        else:
            q["w_r"] = bf16_bits_to_f64(inp["w_r"])
        t0 = time.perf_counter()
        fwd = om.layer_forward(q, wl.k, "bf16")
        om.layer_backward(q, fwd, dy, wl.k, "bf16")
        dt = time.perf_counter() - t0
        log(f"cpu baseline: {Ts} tokens fwd+bwd in {dt:.1f} s")
        if dt >= budget_s or Ts >= wl.T:
            break
        Ts = min(wl.T, Ts * 2)
    return {"value": Ts / dt, "unit": "tokens/s", "cores": threads or cores, "kind": "oracle",
            "sample": f"first {Ts} of {wl.T} tokens of the workload, all {wl.E} experts and full "
                      f"weights, one float64 forward+backward ({dt:.1f} s wall, "
                      f"{cores} host cores visible, {cpu_model()})"}


def cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "CPU model unknown"


def timed(obj, step, steps, warmup, per_step=None):
    """Run `warmup` untimed steps, then time exactly `steps` steps between two
    events on the stream the kernels run on (torch's current stream), with a
    synchronisation on both sides. obj.hook records one event after each
    stage, so stage times come from the same run. Returns (ms per step,
    {stage: mean ms}, wall seconds of the timed region); each step's own ms
    is appended to `per_step` when a list is given."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    marks = []

    def hook(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks.append((name, ev))

    obj.hook = hook
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        hook("_step")
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    obj.hook = None
    stage_ms = {}
    for (_, ea), (b, eb) in zip(marks[:-1], marks[1:]):
        if b == "_step":
            continue
        stage_ms.setdefault(b, []).append(ea.elapsed_time(eb))
    if per_step is not None:
        bounds = [ev for n, ev in marks if n == "_step"] + [end]
        per_step.extend(a.elapsed_time(b) for a, b in zip(bounds[:-1], bounds[1:]))
    return (start.elapsed_time(end) / steps, {n: sum(v) / len(v) for n, v in stage_ms.items()}, wall)


def step_stats(ms):
    """Median, 90th percentile and extremes of the timed steps' own durations."""
    import numpy as np
    a = np.asarray(ms, dtype=float)
    return {"median": round(float(np.median(a)), 4), "p90": round(float(np.percentile(a, 90)), 4),
            "min": round(float(a.min()), 4), "max": round(float(a.max()), 4), "n": int(a.size)}


MALL_BYTES = 256 << 20    # MI355X Infinity Cache (last-level cache in front of HBM)


def weight_residency(wl):
    """Whether the layer's weights (expert and router) could sit in the MALL
    between steps; at E = 128 they cannot, so every step streams them from HBM."""
    w = 3 * wl.E * wl.d * wl.F * 2 + (wl.d * wl.E * 2 if wl.routing == "learned" else 0)
    return {"weight_bytes": w, "mall_bytes": MALL_BYTES, "weights_fit_mall": w <= MALL_BYTES}


def upload_inputs(inp):
    """Host arrays of a workload -> device tensors (bf16 bit patterns kept)."""
    import numpy as np
    import torch
    devc = torch.device("cuda:0")
    t = {}
    for n, a in inp.items():
        a = np.ascontiguousarray(a)
        if n in ("topk_idx", "topk_w", "counts"):
            t[n] = torch.from_numpy(a).to(devc)
        else:
            t[n] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(devc)
    torch.cuda.synchronize()
    return t


def workload_leg(name, capacity_factor, steps, warmup):
    """One bf16 layer forward+backward on another workload of the same
    shape family (its own seeded inputs): step time, grouped-GEMM rate and
    the rows dropped at the given capacity factor (0: dropless)."""
    import torch
    from moe_inputs import make_inputs, workload
    from routing_grouped_expert_router_amd.layer import MoELayer
    wl = workload(name)
    cap = wl.scaled(capacity_factor=capacity_factor).capacity() if capacity_factor > 0 else 0
    t = upload_inputs(make_inputs(wl))
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                     routing="learned" if wl.routing == "learned" else "given", capacity=cap)

    def step():
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                      topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"))
        layer.backward(t["dy"])

    ms, st, _ = timed(layer, step, steps, warmup)
    gemm_ms = sum(v for n, v in st.items() if n.startswith("gg_"))
    counts = layer.counts.cpu().numpy()
    dropped = int(layer.n_dropped.cpu()[0])
    # executed: every row the GEMMs run, pad rows of the padded layout
    # included; useful: only the routed rows that were kept
    executed = 18.0 * layer.n_rows * wl.d * wl.F
    useful = 18.0 * (wl.T * wl.k - dropped) * wl.d * wl.F
    out = {"workload": name, "experts": wl.E, "routing": wl.routing, "capacity": cap,
           "rows": int(layer.n_rows), "tokens_per_s": round(wl.T / (ms / 1e3), 1),
           "ms_per_step": round(ms, 4),
           "grouped_gemm_tflops": round(useful / (gemm_ms / 1e3) / 1e12, 1),
           "grouped_gemm_tflops_executed": round(executed / (gemm_ms / 1e3) / 1e12, 1),
           "expert_load": {"min": int(counts.min()), "max": int(counts.max()),
                           "empty_experts": int((counts == 0).sum())},
           "dropped": dropped}
    del layer, t
    torch.cuda.empty_cache()
    return out


def mx_layer_leg(wl, t, steps, warmup, ms_base):
    """The same routed workload with MXFP8 expert GEMMs and quantise-on-
    dispatch (the permute writes E4M3 rows and scales, never bf16 rows):
    step time and speed-up over the bf16 layer of the main measurement."""
    import torch
    from routing_grouped_expert_router_amd.layer import MoELayer
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                     routing="learned" if wl.routing == "learned" else "given", mxfp8=True,
                     mx_bf16_intermediates=False)

    def step(requantize):
        def run():
            if requantize:   # the weights changed since the last step (one optimiser step per step)
                layer.mx.invalidate_weights()
            layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                          topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"))
            layer.backward(t["dy"])
        return run

    ms, st, _ = timed(layer, step(True), steps, warmup)
    # gradient accumulation: same weights across micro-batches, quantised once
    ms_acc, _, _ = timed(layer, step(False), steps, warmup)
    del layer
    torch.cuda.empty_cache()
    gemm = sum(v for k, v in st.items() if k.startswith("mx_") and not k.startswith("mx_quantize"))
    flops = 18.0 * wl.T * wl.k * wl.d * wl.F
    return {"tokens_per_s": round(wl.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "speedup_vs_bf16": round(ms_base / ms, 3),
            "gemm_tflops": round(flops / (gemm / 1e3) / 1e12, 1),
            "gemm_frac_mxfp8_peak": round(flops / (gemm / 1e3) / 1e12 / PEAK_MXFP8_TFLOPS, 4),
            "weights_unchanged_between_steps": {"tokens_per_s": round(wl.T / (ms_acc / 1e3), 1),
                                                "ms_per_step": round(ms_acc, 4),
                                                "speedup_vs_bf16": round(ms_base / ms_acc, 3)},
            "stages_us": {k: round(v * 1e3, 1) for k, v in st.items()}}


def shared_leg(wl, t, cap, steps, warmup, ms_base):
    """The same workload with one shared expert (d_ff as a routed expert's)
    beside the routed ones: a dense SwiGLU on every token whose output joins
    y in the combine. Inputs of the shared weights are drawn on the device
    from a seeded generator (normal, scaled by fan-in)."""
    import torch
    from routing_grouped_expert_router_amd.layer import MoELayer
    Fs = wl.F
    gen = torch.Generator(device="cuda").manual_seed(wl.seed + 1000)
    rnd = lambda *shape, scale: (torch.randn(*shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    ws = dict(w_gate_s=rnd(wl.d, Fs, scale=wl.d ** -0.5), w_up_s=rnd(wl.d, Fs, scale=wl.d ** -0.5),
              w_down_s=rnd(Fs, wl.d, scale=Fs ** -0.5))
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                     routing="learned" if wl.routing == "learned" else "given", capacity=cap, shared_ff=Fs)

    def step():
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                      topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"), **ws)
        layer.backward(t["dy"])

    ms, st, _ = timed(layer, step, steps, warmup)
    del layer
    torch.cuda.empty_cache()
    sh_us = st.get("gg_shared_fwd", 0.0) + st.get("gg_shared_bwd_data", 0.0) + st.get("gg_shared_bwd_weights", 0.0)
    flops = 18.0 * wl.T * wl.d * Fs
    return {"d_ff_shared": Fs, "tokens_per_s": round(wl.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "shared_gemm_us": round(sh_us * 1e3, 1),
            "shared_gemm_tflops": round(flops / (sh_us / 1e3) / 1e12, 1) if sh_us > 0 else None,
            "step_time_added": round(ms / ms_base - 1.0, 4)}


def memory_probe(wl, t, cap, recompute, n_layers=4):
    """Device memory of the layer under torch's allocator, measured: a stack
    of n_layers independent layers (same weights and inputs) runs every
    forward, then every backward in reverse, as a model does, each layer
    releasing its step's activations and scratch when its backward returns
    (keep_intermediates=False). One warm-up step first allocates the
    gradients (they stay, like parameter gradients). Returns the bytes each
    forward leaves allocated for its backward and the peak of the stack above
    the memory held before the forwards (weights, inputs, gradients)."""
    import torch
    from routing_grouped_expert_router_amd.layer import MoELayer
    layers = [MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                       routing="learned" if wl.routing == "learned" else "given", capacity=cap,
                       recompute=recompute, keep_intermediates=False) for _ in range(n_layers)]
    fwd = lambda lay: lay.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                                  topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"))
    for lay in layers:   # warm-up step: gradients allocated
        fwd(lay)
        lay.backward(t["dy"])
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    held = []
    for lay in layers:
        before = torch.cuda.memory_allocated()
        fwd(lay)
        held.append(torch.cuda.memory_allocated() - before)
    for lay in reversed(layers):
        lay.backward(t["dy"])
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    out = {"held_per_layer_bytes": int(held[-1]), "stack_layers": n_layers,
           "stack_peak_above_resident_bytes": int(peak - base), "stack_peak_bytes": int(peak),
           "resident_bytes": int(base)}
    del layers
    torch.cuda.empty_cache()
    return out


def recompute_leg(wl, t, cap, steps, warmup, ms_base):
    """The same workload with per-layer recompute (the forward writes H
    alone, the backward recomputes G, U and H from x_perm): step time, the
    throughput given up, and the device memory measured under torch's
    allocator with and without recompute (memory_probe)."""
    import torch
    from routing_grouped_expert_router_amd.layer import MoELayer
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                     routing="learned" if wl.routing == "learned" else "given", capacity=cap, recompute=True)

    def step():
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                      topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"))
        layer.backward(t["dy"])

    ms, _, _ = timed(layer, step, steps, warmup)
    del layer
    torch.cuda.empty_cache()
    stored = memory_probe(wl, t, cap, recompute=False)
    recomp = memory_probe(wl, t, cap, recompute=True)
    return {"tokens_per_s": round(wl.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "throughput_cost": round(1.0 - ms_base / ms, 4),
            "memory_stored": stored, "memory_recompute": recomp,
            "activation_memory_saved": round(1.0 - recomp["held_per_layer_bytes"] / stored["held_per_layer_bytes"], 4),
            "stack_peak_above_resident_saved": round(
                1.0 - recomp["stack_peak_above_resident_bytes"] / stored["stack_peak_above_resident_bytes"], 4),
            "stack_peak_saved": round(1.0 - recomp["stack_peak_bytes"] / stored["stack_peak_bytes"], 4)}


def experts_leg(steps, warmup):
    """The MXFP8 expert layer on its own workload (32 experts, d = 4096,
    d_ff = 2048, 32768 rows arriving grouped by expert with Zipf(0.8) counts:
    the pages' expert-parallel microbenchmark shape), timed next to the bf16
    grouped GEMMs on the same rows. A step is every weight quantised in both
    orientations, the forward and the backward of the experts; a second
    timing keeps the weights between steps (gradient accumulation), so they
    are quantised once. Inputs are drawn
    on the device from a seeded generator (normal rows, weights scaled by
    fan-in) so that the leg adds seconds, not minutes, to a run."""
    import numpy as np
    import torch
    from moe_inputs import workload
    from moe_inputs.generators import pregrouped_counts
    from routing_grouped_expert_router_amd.layer import MoELayer
    from routing_grouped_expert_router_amd.mx_layer import MxExperts

    wl = workload("e32_mxfp8_share")
    n, d, E, F = wl.T, wl.d, wl.E, wl.F
    counts = pregrouped_counts(wl.seed, n, E, wl.zipf_s)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    rnd = lambda *shape, scale=1.0: (torch.randn(*shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    x, dy = rnd(n, d), rnd(n, d)
    wg, wu, wd = rnd(E, d, F, scale=d ** -0.5), rnd(E, d, F, scale=d ** -0.5), rnd(E, F, d, scale=F ** -0.5)
    flops = 18.0 * n * d * F

    # H, dG and dU exist only as the MXFP8 copies the next GEMMs read (the
    # bf16 copies are for inspection; the results are the same bits)
    mx = MxExperts(n, d, E, F, bf16_intermediates=False)

    def mx_step(requantize):
        def run():
            if requantize:   # new weights every step
                mx.invalidate_weights()
            mx.forward(x, off, wg, wu, wd)
            mx.backward(dy)
        return run

    ms_mx, st_mx, _ = timed(mx, mx_step(True), steps, warmup)
    gemm_mx = sum(v for k, v in st_mx.items() if not k.startswith("mx_quantize"))
    ms_acc, _, _ = timed(mx, mx_step(False), steps, warmup)
    del mx
    torch.cuda.empty_cache()

    bf = MoELayer(n, d, E, 1, F, torch.bfloat16, routing="given")
    bf.forward_buffers()
    bf.backward_buffers()
    bf.x_perm, bf.offsets, bf.dy_perm = x, off, dy
    bf.w_gate, bf.w_up, bf.w_down = wg, wu, wd

    def bf_step():
        bf.experts_forward()
        bf.experts_backward()

    ms_bf, st_bf, _ = timed(bf, bf_step, steps, warmup)
    del bf
    torch.cuda.empty_cache()
    dom = max((k for k in st_mx if not k.startswith("mx_quantize")), key=st_mx.get)
    dom_flops = {"mx_fwd_gate_up": 4, "mx_fwd_down": 2, "mx_dgrad_down": 2, "mx_dgrad_gate_up": 4,
                 "mx_wgrad_down": 2, "mx_wgrad_gate_up": 4}[dom] * n * d * F
    return {
        "workload": wl.name,
        "config": {"rows": n, "d_model": d, "experts": E, "d_ff": F, "counts_min": int(counts.min()),
                   "counts_max": int(counts.max())},
        "mxfp8_tokens_per_s": round(n / (ms_mx / 1e3), 1),
        "mxfp8_ms_per_step": round(ms_mx, 4),
        "bf16_tokens_per_s": round(n / (ms_bf / 1e3), 1),
        "bf16_ms_per_step": round(ms_bf, 4),
        "mxfp8_speedup": round(ms_bf / ms_mx, 3),
        "mxfp8_gemm_tflops": round(flops / (gemm_mx / 1e3) / 1e12, 1),
        "mxfp8_gemm_frac_peak": round(flops / (gemm_mx / 1e3) / 1e12 / PEAK_MXFP8_TFLOPS, 4),
        "mxfp8_quantize_ms": round(ms_mx - gemm_mx, 4),
        "mxfp8_weights_unchanged_ms_per_step": round(ms_acc, 4),
        "mxfp8_weights_unchanged_speedup": round(ms_bf / ms_acc, 3),
        "roofline": {"bound": "mfma", "kernel": dom, "avg_launch_us": round(st_mx[dom] * 1e3, 1),
                     "achieved": round(dom_flops / (st_mx[dom] / 1e3) / 1e12, 1),
                     "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_flops / (st_mx[dom] / 1e3) / 1e12 / PEAK_MXFP8_TFLOPS, 4)},
        "stages_mxfp8_us": {k: round(v * 1e3, 1) for k, v in st_mx.items()},
        "stages_bf16_us": {k: round(v * 1e3, 1) for k, v in st_bf.items()},
    }


def vendor_gemm_leg(wl, t, steps, warmup):
    """The six expert GEMMs of the layer against hipBLASLt (torch.bmm) on the
    same products with an exactly equal split (every expert T*k/E rows: token
    t's slot j goes to expert (k*t + j) mod E), which a batched product can
    express. Ours run inside the layer step, with their fused epilogues
    (SwiGLU and its derivative, the gate and up halves written apart);
    hipBLASLt's are plain products of contiguous operands into preallocated
    outputs. Both are timed with events over the same number of launches."""
    import torch
    from routing_grouped_expert_router_amd.layer import MoELayer
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    if (T * k) % E:
        return None
    m = T * k // E
    devc = torch.device("cuda:0")
    ids = (torch.arange(T * k, device=devc, dtype=torch.int64) % E).to(torch.int32).view(T, k)
    wts = torch.full((T, k), 1.0 / k, dtype=torch.float32, device=devc)
    layer = MoELayer(T, d, E, k, F, torch.bfloat16, routing="given")

    def step():
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], topk_idx=ids, topk_w=wts)
        layer.backward(t["dy"])

    _, st, _ = timed(layer, step, steps, warmup)
    counts = layer.counts.cpu()
    assert int(counts.min()) == m and int(counts.max()) == m
    del layer
    torch.cuda.empty_cache()
    # (stage, batch operand shapes [E, M, K] x [E, K, N]); flops 2*E*M*K*N
    ops = [("gg_fwd_gate_up", (m, d), (d, 2 * F)), ("gg_fwd_down", (m, F), (F, d)),
           ("gg_dgrad_down", (m, d), (d, F)), ("gg_dgrad_gate_up", (m, 2 * F), (2 * F, d)),
           ("gg_wgrad_down", (F, m), (m, d)), ("gg_wgrad_gate_up", (d, m), (m, 2 * F))]
    g = torch.Generator(device=devc)
    g.manual_seed(7)
    out = {"experts": E, "rows_per_expert": m, "ops": {}}
    ours_us = blas_us = flops_all = 0.0
    for name, (M, K), (K2, N) in ops:
        a = torch.randn(E, M, K, device=devc, generator=g).to(torch.bfloat16)
        b = torch.randn(E, K2, N, device=devc, generator=g).to(torch.bfloat16)
        c = torch.empty(E, M, N, device=devc, dtype=torch.bfloat16)
        for _ in range(warmup):
            torch.bmm(a, b, out=c)
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(steps):
            torch.bmm(a, b, out=c)
        s1.record()
        torch.cuda.synchronize()
        b_us = s0.elapsed_time(s1) / steps * 1e3
        o_us = st[name] * 1e3
        fl = 2.0 * E * M * K * N
        out["ops"][name] = {"ours_us": round(o_us, 1), "ours_tflops": round(fl / o_us / 1e6, 1),
                            "hipblaslt_us": round(b_us, 1), "hipblaslt_tflops": round(fl / b_us / 1e6, 1)}
        ours_us += o_us
        blas_us += b_us
        flops_all += fl
        del a, b, c
    torch.cuda.empty_cache()
    out["ours_tflops"] = round(flops_all / ours_us / 1e6, 1)
    out["hipblaslt_tflops"] = round(flops_all / blas_us / 1e6, 1)
    out["ours_time_vs_hipblaslt"] = round(ours_us / blas_us, 3)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="e128_uniform_bf16")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="> 0: run the padded-to-capacity path")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mxfp8", action="store_true", help="skip the MXFP8 expert-layer leg")
    ap.add_argument("--no-recompute", action="store_true", help="skip the per-layer recompute leg")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-expert leg")
    ap.add_argument("--no-mxfp8-layer", action="store_true", help="skip the MXFP8 routed-layer leg")
    ap.add_argument("--no-pool", action="store_true", help="skip the 8-expert comparison leg")
    ap.add_argument("--no-skew", action="store_true", help="skip the Zipf dropless/padded leg")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the hipBLASLt comparison of the six expert GEMMs on an equal split")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer "
              "is built and timed on a single GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 2, "launches": 3}), flush=True)
        return

    from moe_inputs import make_inputs, workload
    from routing_grouped_expert_router_amd import _lib as L
    from routing_grouped_expert_router_amd.layer import MoELayer

    L.lib()   # fail loudly if the library is missing
    wl = workload(args.workload)
    cap = wl.scaled(capacity_factor=args.capacity_factor).capacity() if args.capacity_factor > 0 else 0
    log(f"generating inputs for {wl.name} ...")
    t0 = time.perf_counter()
    inp = make_inputs(wl)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    t = upload_inputs(inp)
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, torch.bfloat16,
                     routing="learned" if wl.routing == "learned" else "given", capacity=cap)

    def step():
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"),
                      topk_idx=t.get("topk_idx"), topk_w=t.get("topk_w"))
        layer.backward(t["dy"])

    step_ms = []
    ms, stage_avg, wall = timed(layer, step, args.steps, args.warmup, per_step=step_ms)
    n_rows = layer.n_rows
    R = wl.T * wl.k
    gemm_ms = sum(v for n, v in stage_avg.items() if n.startswith("gg_"))
    dropped = int(layer.n_dropped.cpu()[0])
    gemm_flops = 18 * (R - dropped) * wl.d * wl.F        # useful: the kept routed rows
    gemm_flops_executed = 18 * n_rows * wl.d * wl.F      # every row run, pad rows included
    dom = max(stage_avg, key=stage_avg.get)
    kind, work = stage_work(dom, wl, n_rows, R)
    dur_s = stage_avg[dom] / 1e3
    if kind == "mfma":
        achieved = work / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = work / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(stage_avg[dom] * 1e3, 1)
    roof["traffic"] = measured_traffic(dom, wl.name)

    stages = {}
    for n, v in stage_avg.items():
        kd, wk = stage_work(n, wl, n_rows, R)
        s = v / 1e3
        stages[n] = {"us": round(v * 1e3, 1),
                     ("tflops" if kd == "mfma" else "gbs"): round(wk / s / (1e12 if kd == "mfma" else 1e9), 1)}
    counts = layer.counts.cpu().numpy()
    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "experts": wl.E,
                   "top_k": wl.k, "d_ff": wl.F, "routing": wl.routing,
                   "capacity": cap, "parallelism": "single GPU"},
        "roofline": roof,
        "grouped_gemm": {"tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1),
                         "frac_mfma_peak": round(gemm_flops / (gemm_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "tflops_executed": round(gemm_flops_executed / (gemm_ms / 1e3) / 1e12, 1),
                         "ms": round(gemm_ms, 4)},
        "stages": stages,
        "expert_load": {"min": int(counts.min()), "max": int(counts.max()),
                        "mean": float(counts.mean()), "dropped": dropped},
        "step_ms": step_stats(step_ms),
        "memory": weight_residency(wl),
        "wall_s_timed": round(wall, 3),
        "kernel_sources": kernel_source_hash(),
    }
    if not args.no_recompute:
        log("recompute leg ...")
        out["recompute"] = recompute_leg(wl, t, cap, args.steps, args.warmup, ms)
    if not args.no_shared:
        log("shared-expert leg ...")
        out["shared_expert"] = shared_leg(wl, t, cap, args.steps, args.warmup, ms)
    if not args.no_mxfp8_layer and cap == 0:
        log("MXFP8 routed-layer leg ...")
        out["mxfp8_layer"] = mx_layer_leg(wl, t, args.steps, args.warmup, ms)
    if not args.no_mxfp8:
        log("MXFP8 expert-layer leg ...")
        out["mxfp8_experts"] = experts_leg(args.steps, args.warmup)
    if not args.no_pool and wl.name == "e128_uniform_bf16" and cap == 0:
        # the same layer with 8 experts (uniform routing, same T, d, k, d_ff),
        # and the 8-expert learned-router configuration
        log("expert-pool leg (E = 8) ...")
        e8 = workload_leg("e8_uniform_bf16", 0.0, args.steps, args.warmup)
        e8l = workload_leg("e8_learned_bf16", 0.0, args.steps, args.warmup)
        out["expert_pool"] = {"e8_uniform": e8, "e8_learned": e8l,
                              "throughput_loss_e8_to_e128": round(1.0 - out["value"] / e8["tokens_per_s"], 4)}
    if not args.no_skew:
        log("skewed-routing leg (dropless and padded) ...")
        dl = workload_leg("e128_zipf_bf16", 0.0, args.steps, args.warmup)
        pd = workload_leg("e128_zipf_bf16", 1.25, args.steps, args.warmup)
        out["skewed_routing"] = {"dropless": dl, "padded_cf1.25": pd,
                                 "padded_time_vs_dropless": round(pd["ms_per_step"] / dl["ms_per_step"], 3)}
    if not args.no_vendor and cap == 0:
        log("vendor GEMM leg (hipBLASLt on the equal split) ...")
        out["vendor_gemm"] = vendor_gemm_leg(wl, t, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host for the CPU baseline ...")
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
