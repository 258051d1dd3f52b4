"""Benchmark of the routed-MoE decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload glm_t1] [--split]

A step is one pass of the whole path (route -> gate/up + SwiGLU -> down +
combine) over one batch of synthetic tokens; the default workload is one
GLM-5.2-shaped layer (hidden 6144, expert intermediate 2048, 256 routed experts
in 8 groups, top-4 groups, top-8, one shared expert, int4 codes with fp32 row
scales) decoding one token.  Several such layers are resident in HBM and the
steps rotate over them and over a pool of 64 tokens.  The step is the
single-launch fused call where its limits allow (--split: the three separate
calls).  Prints one JSON line.

Headline timing (the flushed protocol): before every step a 1 GiB buffer is
read (outside the timed region), so neither the L2s nor the 256 MB Infinity
Cache hold any of the step's data; HIP events on the step's stream bracket
each step.  (A write of 1 GiB instead leaves dirty lines whose write-back then
competes with the step: that figure is reported apart as `write_flush`.)  `value` = the bytes of all timed steps / the sum of their
event-timed durations; `ms_per_step` their mean.  Secondary figures: the same
steps replayed back to back from HIP graphs with no flush (`no_flush`), and a
plain 128-bit streaming read of the same bytes and of 4 GiB (`read_ceiling`,
the achievable read rate the step is also quoted against).

Bytes per step (the metric's count) = the unique selected experts' packed
codes and row scales + the input and output activations; the router weight is
excluded and reported apart.  The roofline object prices the fused launch by
those same bytes over its event-timed duration.
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

METRIC = "achieved HBM GB/s (% of peak) and tokens/s for one int4 256-expert MoE layer"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "quantized_moe_decode_route_amd", "csrc")
# sources each timed kernel is built from (the traffic counters are void once any changes)
KERNEL_SRCS = {"fused": ["layer_pipe.hip", "imma.h", "persist.h", "route.h", "common.h"],
               "gate_up": ["experts_mfma.hip", "mfma.h", "persist.h", "common.h"],
               "quantize": ["quant.hip", "common.h"]}


def step_bytes(cfg, n_active: int) -> int:
    return n_active * cfg.expert_bytes() + 2 * cfg.tokens * cfg.hidden * 4


def router_bytes(cfg) -> int:
    return cfg.n_experts * cfg.hidden * 4


def fused_bytes(cfg, n_active: int) -> int:
    """Algorithmic bytes of one fused launch: the step bytes, the router weight
    and bias read, the scores and h written."""
    return (step_bytes(cfg, n_active) + router_bytes(cfg) + cfg.n_experts * 4 + cfg.tokens * cfg.n_experts * 4
            + cfg.tokens * cfg.slots * cfg.inter * 4)


def gate_up_bytes(cfg, n_active: int) -> int:
    """Algorithmic bytes of one gate/up launch: gate and up codes and scales of
    the active experts, the activations read and h written."""
    per = 2 * cfg.inter * (cfg.hidden * cfg.bits // 8 + 4)
    return n_active * per + cfg.tokens * cfg.hidden * 4 + cfg.tokens * cfg.slots * cfg.inter * 4


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SRCS[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kind: str, workload: str):
    """HBM bytes per launch of the timed kernel measured with rocprofv3
    counters, if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f).get(kind, {}).get(workload, {})
    except (OSError, ValueError, AttributeError):
        return None
    if d.get("kernel_sha") != kernel_hash(kind):
        return None
    return d.get("bytes_per_launch")


def host_cores() -> dict:
    """The host CPU the oracle runs on: logical CPUs this process may use and the model name."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"usable_cpus": usable, "os_cpu_count": os.cpu_count(), "model": model}


def cpu_baseline(cfg, budget_s: float, top_p: float | None = None, act8: bool = False) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload, at
    one thread and at every usable core.  The plain-C implementation
    (oracle/moe_ref.c, OpenMP over rows) is the one timed; the top-p and
    int8-activation variants exist only in the NumPy oracle, which then runs
    on one thread."""
    from oracle import moe_oracle as orc
    from quantized_moe_decode_route_amd import synth

    host = host_cores()
    if top_p is not None or act8:
        return cpu_baseline_numpy(cfg, budget_s, top_p, act8, host)
    from oracle import moe_ref

    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    experts, tokens = {}, []
    # the layer is resident: the experts the sample's tokens select are generated before timing
    n_tok = max(2, min(cfg.pool, 32))
    for i in range(n_tok):
        x = synth.batch_tokens(cfg, i)
        s64 = orc.router_scores(x, rw)
        idx, _ = orc.select_experts(s64.astype(np.float32), b, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rsf)
        for e in set(idx.ravel().tolist()) | set(range(cfg.n_experts, cfg.n_experts + cfg.n_shared)):
            if e not in experts:
                experts[e] = synth.expert_arrays(cfg, 0, e)
        tokens.append((x, len(set(idx.ravel().tolist())) + cfg.n_shared))
    kw = dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, n_shared=cfg.n_shared, rsf=cfg.rsf,
              bits=cfg.bits)

    def timed(threads: int, budget: float) -> dict:
        elapsed, nbytes, ntok, steps = 0.0, 0, 0, 0
        while steps < len(tokens) and (elapsed < budget or steps == 0):
            x, n_act = tokens[steps]
            t0 = time.perf_counter()
            moe_ref.layer(x, rw, b, experts, threads=threads, **kw)
            elapsed += time.perf_counter() - t0
            nbytes += step_bytes(cfg, n_act)
            ntok += cfg.tokens
            steps += 1
        return {"gbs": nbytes / elapsed / 1e9, "tok_s": ntok / elapsed, "steps": steps, "seconds": elapsed}

    n_all = host["usable_cpus"]
    one = timed(1, budget_s * 0.6)
    full = timed(n_all, budget_s * 0.4)
    return {"value": round(full["gbs"], 4), "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "tokens_per_s": round(full["tok_s"], 4),
            "single_thread": {"value": round(one["gbs"], 4), "unit": "GB/s", "cores": 1,
                              "tokens_per_s": round(one["tok_s"], 4)},
            "host": host,
            "sample": f"plain-C oracle (OpenMP over rows, fp64 expert arithmetic) on {cfg.name}, layer 0: "
                      f"{full['steps']} steps on {n_all} threads in {full['seconds']:.1f} s and {one['steps']} steps "
                      f"on 1 thread in {one['seconds']:.1f} s (router over all experts + the selected experts; "
                      f"input generation excluded)"}


def cpu_baseline_numpy(cfg, budget_s: float, top_p: float | None, act8: bool, host: dict) -> dict:
    """The NumPy oracle on one thread (the top-p and int8-activation variants)."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as orc
    from quantized_moe_decode_route_amd import synth

    layers = 4
    data = {}
    elapsed, nbytes, ntok, steps = 0.0, 0, 0, 0
    with threadpool_limits(limits=1):
        while steps < 64 and (elapsed < budget_s or steps == 0):
            l = steps % layers
            if l not in data:
                data[l] = (synth.router_weight(cfg, l), synth.router_bias(cfg, l), {})
            rw, b, cache = data[l]
            x = synth.batch_tokens(cfg, steps)
            # the layer is resident: fetch the experts this step needs before timing
            s64 = orc.router_scores(x, rw)
            idx, _ = orc.select_experts(s64.astype(np.float32), b, cfg.n_group, cfg.topk_group, cfg.top_k,
                                        cfg.rsf)
            need = set(idx.ravel().tolist()) | set(range(cfg.n_experts, cfg.n_experts + cfg.n_shared))
            for e in need:
                if e not in cache:
                    cache[e] = synth.expert_arrays(cfg, l, e)
            t0 = time.perf_counter()
            r = orc.moe_layer(x, rw, b, cache.__getitem__, n_group=cfg.n_group, topk_group=cfg.topk_group,
                              top_k=cfg.top_k, n_shared=cfg.n_shared, rsf=cfg.rsf, bits=cfg.bits,
                              top_p=1.0 if top_p is None else top_p, act8=act8)
            elapsed += time.perf_counter() - t0
            nbytes += step_bytes(cfg, len(r.worklist.expert_id))
            ntok += cfg.tokens
            steps += 1
            if len(cache) > 40:
                cache.clear()
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": round(ntok / elapsed, 4), "host": host,
            "sample": f"NumPy oracle: {steps} steps ({ntok} tokens) of {cfg.name} on {layers} rotating layers, "
                      f"{elapsed:.1f} s of oracle time, 1 thread"}


# The pages' own figures: whole-model GLM-5.2 decode on CPUs with experts
# streamed from disk -- context for the tokens/s above, not the same workload.
PAGES_CONTEXT = {
    "note": "whole-model CPU/disk decode figures from the pages; a different workload from one resident layer",
    "cold_decode_tok_s": [0.05, 0.1],
    "cold_decode_setup": "12-core WSL2 machine, 25 GB RAM, experts read from NVMe (~11 GB per token), int4",
    "m5_max_tok_s": 1.06,
    "m5_max_setup": "Apple M5 Max, 18 cores, 128 GB unified memory, MTP off, int4",
}


def fused_kernel_name(cfg, top_p, act8: bool, resid: bool) -> str:
    """The kernel a fused call launches (as the profiler names it)."""
    tp = "true" if top_p is not None and top_p < 1 else "false"
    if act8:
        ncb = 2 if cfg.bits == 8 else 4               # MFMA columns of a token (one per column block)
        passes = 1 if cfg.tokens * ncb <= 16 else ncb
        return f"layer_fused_kernel<{cfg.bits}, {tp}, false, true, {passes}>"
    np_ = 1 if 3 * cfg.tokens <= 16 else 3
    return f"layer_pipe_kernel<{cfg.bits}, {np_}, {tp}, {'true' if resid else 'false'}>"


def step_dtype(bits: int, fused: bool, act8: bool) -> str:
    """The arithmetic the timed step computes in."""
    if act8:
        return f"int{bits} codes x int8 activation blocks -> int32, fp32 block scales and sums"
    if fused:
        return f"int{bits} codes x int24 activations -> exact int32, fp32 scales and sums"
    return f"int{bits} codes -> f16, f16 hi/lo activations, fp32 accumulate"


def quantize_bytes(rows: int, n: int, bits: int) -> int:
    """Algorithmic bytes of one quantiser launch: the fp32 rows read once, the
    packed codes and the row scales written once."""
    return rows * n * 4 + rows * n * bits // 8 + rows * 4


def bench_quantize(args) -> None:
    """The row quantiser on GLM-5.2 expert matrices: int4, packed output, one
    launch per matrix ([4096, 6144] gate+up rows, [6144, 2048] down rows),
    rotating over 8 experts' fp32 matrices (1.2 GB) so no launch finds its input
    in the caches; a step is one launch.  Prints one JSON line of its own."""
    import torch

    from quantized_moe_decode_route_amd import ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bits, n_exp = 4, 8
    shapes = [(4096, 6144), (6144, 2048)]
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    mats, outs, scl = [], [], []
    for e in range(n_exp):
        for rows, n in shapes:
            w = torch.randn((rows, n), generator=g, device=dev) * 0.02
            mats.append(w)
            outs.append(torch.empty((rows, n * bits // 8), dtype=torch.uint8, device=dev))
            scl.append(torch.empty(rows, dtype=torch.float32, device=dev))
    # per matrix shape: one HIP graph of the 8 experts' launches, replayed
    # back to back; the launch average is the event-timed region / launches
    stream = torch.cuda.Stream()
    reps = max(args.steps // 160, 4)
    per, tot_bytes, tot_s, launches = {}, 0, 0.0, 0
    for si, (rows, n) in enumerate(shapes):
        idx = [e * len(shapes) + si for e in range(n_exp)]
        with torch.cuda.stream(stream):
            for k in idx:
                ops.quantize_rows(mats[k], bits, pack=True, out=outs[k], scales=scl[k])
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for k in idx:
                ops.quantize_rows(mats[k], bits, pack=True, out=outs[k], scales=scl[k])
        with torch.cuda.stream(stream):
            graph.replay()
            ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev_a.record(stream)
            for _ in range(reps):
                graph.replay()
            ev_b.record(stream)
        stream.synchronize()
        region = ev_a.elapsed_time(ev_b) * 1e-3
        nl = reps * n_exp
        b = quantize_bytes(rows, n, bits)
        per[f"{rows}x{n}"] = {"avg_us": round(region / nl * 1e6, 2), "gbs": round(b * nl / region / 1e9, 1),
                              "bytes_per_launch": b}
        tot_bytes += b * nl
        tot_s += region
        launches += nl
    value = tot_bytes / tot_s / 1e9
    print(f"[bench] quantiser: {launches} launches, {value:.0f} GB/s ({per})", file=sys.stderr, flush=True)
    # the dominant kernel: the gate/up-shaped launch (2/3 of the bytes)
    dom = per["4096x6144"]
    achieved = dom["bytes_per_launch"] / (dom["avg_us"] * 1e-6) / 1e9

    base = None
    if args.cpu_budget > 0:
        from threadpoolctl import threadpool_limits

        from oracle import moe_oracle as orc
        w = mats[0][:256].cpu().numpy()
        t_used, nbytes, reps = 0.0, 0, 0
        with threadpool_limits(limits=1):
            while t_used < min(args.cpu_budget, 10.0) or reps == 0:
                t0 = time.perf_counter()
                orc.pack_rows(orc.quantize_rows(w, bits)[0], bits)
                t_used += time.perf_counter() - t0
                nbytes += quantize_bytes(w.shape[0], w.shape[1], bits)
                reps += 1
        base = {"value": round(nbytes / t_used / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{reps} x 256 rows of 6144 fp32 -> packed int4, {t_used:.1f} s, 1 thread"}

    out = {
        "metric": "row quantiser achieved HBM GB/s (fp32 expert matrices -> packed int4 codes + row scales)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": launches, "warmup": len(shapes) * n_exp,
        "ms_per_step": round(tot_s / launches * 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 rows -> int4 codes (fp32 division, round half to even)",
        "data": "synthetic",
        "config": {"workload": "glm_expert_matrices_q4", "matrices": [list(s) for s in shapes], "experts": n_exp,
                   "bits": bits, "output": "packed"},
        "roofline": {"bound": "hbm", "kernel": "quantize_rows_cached<4, true, 4, 6> (4096 x 6144)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("quantize", "glm_expert_matrices_q4"),
                     "avg_us": dom["avg_us"], "bytes_per_launch": dom["bytes_per_launch"], "per_shape": per},
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


def bench_stack(args, cfg) -> None:
    """A stack of cfg.layers resident layers (x <- x + MoE(rmsnorm(x)) per
    layer, the pre-norm residual form) on cfg.tokens tokens; a step is the
    whole stack, captured as one HIP graph per token batch and replayed.
    Bytes per step = the per-layer step bytes summed over the layers."""
    import torch

    from quantized_moe_decode_route_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, H, L = cfg.tokens, cfg.hidden, cfg.layers
    kw = dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)
    layers, experts = [], []
    for l in range(L):
        layers.append(synth.layer_device(cfg, l, dev))
        experts.append(ops.Experts.from_layer(layers[-1], cfg.n_experts, cfg.n_shared, cfg.bits))
        print(f"[bench] layer {l} resident", file=sys.stderr, flush=True)
    bufs = [ops.LayerBuffers.allocate(T, H, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared, dev) for _ in range(L)]
    n_batch = cfg.pool // T
    pool = torch.from_numpy(synth.token_pool(cfg)).to(dev)
    x = torch.empty((T, H), dtype=torch.float32, device=dev)
    xn = torch.empty_like(x)
    stack = [(lay["router_w"], lay["bias"], ex) for lay, ex in zip(layers, experts)]
    # fused: one residual-form launch per layer (norm and residual inside);
    # else the separate calls with the norm kernel between layers
    fused = ops.stack_forward(x.copy_(pool[:T]), stack, bufs, top_p=args.top_p, xn=xn, **kw)

    def step(b):
        x.copy_(pool[b * T:(b + 1) * T])
        ops.stack_forward(x, stack, bufs, top_p=args.top_p, fused=fused, xn=xn, **kw)

    # unique experts per layer for each token batch (routing depends on the batch only)
    sbytes = np.zeros(n_batch)
    active = np.zeros((n_batch, L), np.int64)
    for b in range(n_batch):
        step(b)
        torch.cuda.synchronize()
        for l in range(L):
            active[b, l] = int(bufs[l].route.worklist.n_active.item())
        sbytes[b] = sum(step_bytes(cfg, int(n)) for n in active[b])
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        step(0)
    stream.synchronize()
    for b in range(n_batch):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(b)
        graphs.append(g)
    steps, warm = max(args.steps // 100, 8), max(args.warmup // 100, 2)
    for i in range(warm):
        graphs[i % n_batch].replay()
    torch.cuda.synchronize()
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev_a.record()
    for i in range(steps):
        graphs[(warm + i) % n_batch].replay()
    ev_b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = ev_a.elapsed_time(ev_b) * 1e-3
    idx = (np.arange(warm, warm + steps) % n_batch)
    total = float(sbytes[idx].sum())
    gbs = total / wall / 1e9
    print(f"[bench] {steps} stack steps in {wall * 1e3:.1f} ms (events {region * 1e3:.1f} ms): "
          f"{wall / steps * 1e3:.3f} ms/step, {gbs:.0f} GB/s, {steps * T / wall:.0f} tok/s through {L} layers; "
          f"unique experts per layer {active.mean():.1f}", file=sys.stderr, flush=True)

    # the dominant kernel (gate/up of the split path, or the fused launch), timed
    # eagerly with HIP events per launch, each after a read of a 1 GiB buffer
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
    kb = []
    for k in range(2 * L):
        l, b = k % L, (k // L) % n_batch
        x.copy_(pool[b * T:(b + 1) * T])
        ops.residual_rmsnorm(x, None, xn)
        sink += flush.sum()
        if fused:
            ev0[k].record()
            ops.layer_fused(x, layers[l]["router_w"], layers[l]["bias"], experts[l], buf=bufs[l],
                            top_p=args.top_p, x_out=xn, **kw)
            ev1[k].record()
            kb.append(fused_bytes(cfg, int(bufs[l].route.worklist.n_active.item())))
        else:
            ops.route_topk(xn, layers[l]["router_w"], layers[l]["bias"], n_shared=cfg.n_shared, out=bufs[l].route,
                           top_p=args.top_p, **kw)
            ev0[k].record()
            ops.gate_up_silu(xn, experts[l], bufs[l].route.worklist, cfg.top_k, out=bufs[l].h)
            ev1[k].record()
            kb.append(gate_up_bytes(cfg, int(bufs[l].route.worklist.n_active.item())))
    torch.cuda.synchronize()
    dur = np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)]) * 1e-3
    achieved = float(np.mean(kb) / dur.mean() / 1e9)
    kname = fused_kernel_name(cfg, args.top_p, False, True) if fused else f"gate_up_mfma_kernel<{cfg.bits}>"
    print(f"[bench] {kname} avg {dur.mean() * 1e6:.1f} us, {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    traffic = traffic_from_profile("fused" if fused else "gate_up", cfg.name) if args.top_p is None else None
    base = cpu_baseline(cfg, args.cpu_budget, args.top_p) if args.cpu_budget > 0 else None
    out = {
        "metric": METRIC + " (16-layer stack)", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(wall / steps * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": step_dtype(cfg.bits, fused, False), "data": "synthetic",
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "tokens_per_s": round(steps * T / wall, 1),
        "bytes_per_step": int(sbytes[idx].mean()),
        "config": {"workload": cfg.name, "path": "fused" if fused else "split", "tokens": T, "layers": L,
                   "hidden": H, "inter": cfg.inter, "routed_experts": cfg.n_experts, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "top_k": cfg.top_k, "shared_experts": cfg.n_shared,
                   "bits": cfg.bits, "zipf_bias": cfg.zipf_s, "graph": "one per step over every layer",
                   "layer_form": "one residual-form fused launch per layer" if fused else
                   "separate calls + residual/RMSNorm kernel per layer",
                   "unique_experts_per_layer": float(active[idx].mean()), "top_p": args.top_p},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_us": round(float(dur.mean() * 1e6), 2), "bytes_per_launch": int(np.mean(kb))},
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="glm_t1")
    ap.add_argument("--layers", type=int, default=4, help="resident layers the steps rotate over")
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's batch (stack workloads)")
    ap.add_argument("--graph-steps", type=int, default=8)
    ap.add_argument("--kernel-steps", type=int, default=20, help="flushed gate/up launches timed (split path)")
    ap.add_argument("--split", action="store_true", help="time the three separate calls instead of the fused one")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="route with adaptive expert top-p at this p (moe_layer_fused_topp / moe_route_topp)")
    ap.add_argument("--act8", action="store_true",
                    help="the fused layer with Q8_0-style int8 activations (moe_layer_fused_act8)")
    ap.add_argument("--quantize", action="store_true",
                    help="time the row quantiser instead (fp32 expert matrices -> packed codes + row scales)")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the streaming-read ceiling (moe_bench_stream_read)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB 20 times (a known-size "
                         "reference for the HBM traffic counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_moe_decode_route_amd import ops, synth

    if args.copy_mib > 0:
        n = args.copy_mib << 18                      # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "copies": 20}), flush=True)
        return

    if args.quantize:
        bench_quantize(args)
        return

    cfg = synth.CONFIGS[args.workload]
    if args.tokens is not None:
        if cfg.layers == 1:
            raise SystemExit("--tokens applies to the stack workloads only")
        cfg = synth.scaled(cfg, tokens=args.tokens, name=f"{cfg.name}_t{args.tokens}")
    if cfg.layers != 1:
        bench_stack(args, cfg)
        return
    bench_layer(args, cfg)


class Flusher:
    """Empties the L2s and the 256 MB Infinity Cache of a step's data before
    the step, outside its timed region.  mode "read": a plain streaming read
    of 1 GiB (moe_bench_stream_read), which leaves only clean lines behind;
    mode "write": 1 GiB written (torch fill), which leaves dirty lines that the
    next kernel's reads must evict -- write-backs that then share HBM with
    that kernel (reported apart, not the headline)."""

    def __init__(self, dev, mode: str, mib: int = 1024):
        import torch

        self.mode = mode
        self.buf = torch.ones(mib << 18, dtype=torch.float32, device=dev)
        cu = torch.cuda.get_device_properties(dev).multi_processor_count
        self.grid = 2 * cu
        self.sink = torch.zeros(self.grid * 512, dtype=torch.int32, device=dev)

    def __call__(self, k: int) -> None:
        from quantized_moe_decode_route_amd import ops

        if self.mode == "write":
            self.buf.fill_(float(k))
        else:
            ops.stream_read(self.buf, self.sink, self.grid, 512, 8)


def flushed_times(step, n_warm: int, n_steps: int, dev, mode: str = "read") -> np.ndarray:
    """The flushed protocol: before each step a flush (outside the timed
    region), then HIP events on the current stream around the step.  Returns
    the event-timed seconds of the n_steps steps after n_warm warm-up steps.
    The flush takes long enough that the host has enqueued the step and its
    events before the GPU reaches them."""
    import torch

    flush = Flusher(dev, mode)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
    for i in range(n_warm):
        flush(i)
        step(i)
    torch.cuda.synchronize()
    for k in range(n_steps):
        flush(k)
        ev0[k].record()
        step(n_warm + k)
        ev1[k].record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)]) * 1e-3


def read_ceiling(dev, step_nbytes: int) -> dict:
    """A plain 128-bit streaming read (moe_bench_stream_read): the best rate
    over a few launch shapes on 4 GiB, and the time to read one step's bytes
    from a region not read since the last (read) flush."""
    import torch

    from quantized_moe_decode_route_amd import ops

    big = 4 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device=dev)
    flush = Flusher(dev, "read")
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    shapes = [(g * cu, th, u) for g in (1, 2, 4, 8) for th in (256, 512) for u in (8, 16) if g * th <= 4096]
    sink = torch.zeros(max(g * th for g, th, _ in shapes), dtype=torch.int32, device=dev)
    best, sweep = None, {}
    for g, th, u in shapes:
        ops.stream_read(buf, sink, g, th, u)          # warm the code path
        ts = []
        for k in range(3):
            flush(k)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ops.stream_read(buf, sink, g, th, u)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        gbs = big / min(ts) / 1e9
        sweep[f"{g}x{th}x{u}"] = round(gbs, 1)
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "grid": g, "threads": th, "unroll": u}
    # one step's bytes, from a rotating region, flushed before each read
    nb = (step_nbytes + 15) // 16 * 16
    per = max(1, big // nb - 1)
    small = []
    for shape in ((cu, 512, 8), (best["grid"], best["threads"], best["unroll"])):
        ts = []
        for k in range(8):
            flush(k)
            off = (k % per) * nb // 4
            view = buf[off:off + nb // 4]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ops.stream_read(view, sink, shape[0], shape[1], shape[2])
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        small.append((float(np.median(ts[1:])), shape))
    t_step, shape = min(small)
    del buf
    return {"gbs": best["gbs"], "pct_of_peak": round(100 * best["gbs"] / HBM_PEAK_GBS, 1), "config": best,
            "bytes": big, "step_bytes": nb, "step_bytes_us": round(t_step * 1e6, 2),
            "step_bytes_gbs": round(nb / t_step / 1e9, 1),
            "step_bytes_config": {"grid": shape[0], "threads": shape[1], "unroll": shape[2]},
            "sweep_gbs": sweep, "kernel": "stream_read_kernel (moe_bench_stream_read), read-flushed before each launch"}


def bench_layer(args, cfg) -> None:
    """One resident layer: flushed per-step timing (the headline), graph
    replays without flush, the read ceiling, the roofline and the CPU baseline."""
    import torch

    from quantized_moe_decode_route_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, T, G = args.layers, cfg.tokens, args.graph_steps
    layers = [synth.layer_device(cfg, l, dev) for l in range(L)]
    experts = [ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits) for lay in layers]
    pool = torch.from_numpy(synth.token_pool(cfg)).to(dev)
    n_pool = cfg.pool
    period = int(np.lcm(L, n_pool))
    kw = dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)
    bufs = [ops.LayerBuffers.allocate(T, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared, dev)
            for _ in range(L)]

    def tokens(i):
        b = i % n_pool
        return pool[b * T:(b + 1) * T]

    fused = (not args.split) and ops.fused_supported(T, experts[0])
    if fused:
        try:
            ops.layer_fused(tokens(0), layers[0]["router_w"], layers[0]["bias"], experts[0], buf=bufs[0],
                            top_p=args.top_p, act8=args.act8, **kw)
        except ops.MoedecError as err:
            if err.status != ops.MOEDEC_ERR_UNSUPPORTED:
                raise
            fused = False            # the batch does not fit the fused call's LDS plan

    def step(i, check=None):
        l = i % L
        ops.moe_layer(tokens(i), layers[l]["router_w"], layers[l]["bias"], experts[l], buf=bufs[l], fused=fused,
                      top_p=args.top_p, act8=args.act8, check=check, **kw)

    # unique experts of every step of the period (routing is a function of (layer, token))
    n_active = np.zeros(period, np.int64)
    for i in range(period):
        step(i)
        torch.cuda.synchronize()
        n_active[i] = int(bufs[i % L].route.worklist.n_active.item())
    sbytes = np.array([step_bytes(cfg, int(n)) for n in n_active])

    # ---- headline: flushed steps, each bracketed by events
    first = args.warmup
    idx = (np.arange(first, first + args.steps) % period)
    t0 = time.perf_counter()
    dur = flushed_times(lambda i: step(i, check=False), args.warmup, args.steps, dev, "read")
    wall = time.perf_counter() - t0
    wdur = flushed_times(lambda i: step(i, check=False), 2, min(args.steps, 10), dev, "write")
    if fused:
        for b in bufs:
            b.check_fused()
    total_bytes = float(sbytes[idx].sum())
    gbs = total_bytes / dur.sum() / 1e9
    ms_per_step = float(dur.mean() * 1e3)
    tok_s = args.steps * T / dur.sum()
    print(f"[bench] flushed: {args.steps} steps, {ms_per_step * 1e3:.2f} us/step (median "
          f"{np.median(dur) * 1e6:.2f}), {gbs:.0f} GB/s, {tok_s:.0f} tok/s; timed region with flushes "
          f"{wall * 1e3:.1f} ms", file=sys.stderr, flush=True)

    # ---- secondary: graph replays back to back, rotating layers and tokens, no flush
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    blocks = {}
    with torch.cuda.stream(stream):
        for i in range(3):
            step(i)
    stream.synchronize()
    for i0 in range(0, period, G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(i0, i0 + G):
                step(i)
        blocks[i0] = g
    n_rep = max(1, (args.steps + args.warmup + G - 1) // G)
    reps = [blocks[(k * G) % period] for k in range(n_rep + 2)]
    with torch.cuda.stream(stream):
        reps[0].replay()
        reps[1].replay()
        ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev_a.record(stream)
        for g in reps[2:]:
            g.replay()
        ev_b.record(stream)
    stream.synchronize()
    nf_s = ev_a.elapsed_time(ev_b) * 1e-3
    nf_steps = n_rep * G
    nf_idx = (np.arange(2 * G, 2 * G + nf_steps) % period)
    nf_bytes = float(sbytes[nf_idx].sum())
    no_flush = {"gbs": round(nf_bytes / nf_s / 1e9, 1), "us_per_step": round(nf_s / nf_steps * 1e6, 2),
                "tokens_per_s": round(nf_steps * T / nf_s, 1), "steps": nf_steps,
                "method": f"HIP graphs of {G} consecutive steps replayed back to back, rotating over {L} layers "
                          f"and {n_pool} token batches, no cache flush"}
    print(f"[bench] no flush: {no_flush['us_per_step']} us/step, {no_flush['gbs']} GB/s; after a 1 GiB write: "
          f"{wdur.mean() * 1e6:.2f} us/step", file=sys.stderr, flush=True)
    write_flush = {"us_per_step": round(float(wdur.mean() * 1e6), 2), "steps": len(wdur),
                   "note": "1 GiB written before each step instead of read: the dirty lines it leaves are written "
                           "back while the step streams its weights"}
    if fused:
        for b in bufs:
            b.check_fused()

    ceiling = read_ceiling(dev, int(np.mean(sbytes[idx]))) if args.ceiling else None
    if ceiling:
        print(f"[bench] read ceiling: {ceiling['gbs']} GB/s on 4 GiB; one step's bytes in "
              f"{ceiling['step_bytes_us']} us ({ceiling['step_bytes_gbs']} GB/s)", file=sys.stderr, flush=True)

    # ---- the dominant kernel: the fused launch is the whole step; the split
    # path's gate/up launch is timed on its own, flushed the same way
    kind = "fused" if fused else "gate_up"
    if fused:
        kdur = dur
        kb = [int(b) for b in sbytes[idx]]
    else:
        def gu(i):
            l = i % L
            ops.route_topk(tokens(i), layers[l]["router_w"], layers[l]["bias"], n_shared=cfg.n_shared,
                           out=bufs[l].route, top_p=args.top_p, **kw)

        kb, times = [], []
        flush = Flusher(dev, "read")
        for k in range(args.kernel_steps):
            i = first + k
            l = i % L
            gu(i)
            flush(k)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ops.gate_up_silu(tokens(i), experts[l], bufs[l].route.worklist, cfg.top_k, out=bufs[l].h)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
            kb.append(gate_up_bytes(cfg, int(n_active[i % period])))
        kdur = np.array(times)
    achieved = float(np.mean(kb) / kdur.mean() / 1e9)
    traffic = traffic_from_profile(kind, cfg.name) if args.top_p is None and not args.act8 else None
    kname = fused_kernel_name(cfg, args.top_p, args.act8, False) if fused else f"gate_up_mfma_kernel<{cfg.bits}>"
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "avg_us": round(float(kdur.mean() * 1e6), 2),
                "median_us": round(float(np.median(kdur) * 1e6), 2),
                "bytes_per_launch": int(np.mean(kb)),
                "bytes_rule": "unique selected experts' codes + row scales + x in + y out (router excluded)" if fused
                else "gate/up codes + row scales of the active experts + x in + h out",
                "timing": "HIP events around each launch on its stream, 1 GiB read before each (flushed)"}
    if ceiling:
        roofline["frac_of_read_ceiling"] = round(achieved / ceiling["gbs"], 4)
    print(f"[bench] {kname} avg {kdur.mean() * 1e6:.2f} us, {achieved:.0f} GB/s", file=sys.stderr, flush=True)

    base = cpu_baseline(cfg, args.cpu_budget, args.top_p, args.act8) if args.cpu_budget > 0 else None

    p10, p50, p90 = (float(np.percentile(dur, q) * 1e6) for q in (10, 50, 90))
    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": step_dtype(cfg.bits, fused, args.act8),
        "data": "synthetic",
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "tokens_per_s": round(tok_s, 1),
        "pct_of_read_ceiling": round(100 * gbs / ceiling["gbs"], 2) if ceiling else None,
        "step_us": {"mean": round(ms_per_step * 1e3, 2), "p10": round(p10, 2), "median": round(p50, 2),
                    "p90": round(p90, 2)},
        "timing": "flushed: 1 GiB read before each step (outside the timed region), HIP events around the step; "
                  "value = bytes of all timed steps / sum of their durations",
        "bytes_per_step": int(sbytes[idx].mean()), "router_bytes_per_step": router_bytes(cfg),
        "config": {"workload": cfg.name, "path": "fused" if fused else "split", "tokens": T, "hidden": cfg.hidden,
                   "inter": cfg.inter, "routed_experts": cfg.n_experts, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "top_k": cfg.top_k, "shared_experts": cfg.n_shared,
                   "bits": cfg.bits, "resident_layers": L, "unique_experts_per_step": float(n_active[idx].mean()),
                   "top_p": args.top_p},
        "no_flush": no_flush, "write_flush": write_flush, "read_ceiling": ceiling,
        "roofline": roofline, "cpu_baseline": base, "context": PAGES_CONTEXT,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
