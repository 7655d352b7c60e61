#!/usr/bin/env python3
"""MoE-stack decode benchmark on one MI355X: tokens/s at batch 1 and achieved HBM GB/s.

Default workload: the 40-layer bf16 stack shaped like Qwen3.5-35B-A3B -- H=2048, E=256
routed experts, top-8 with softmax over the selected logits, one always-on shared expert,
expert width I=768 -- with synthetic N(0, 0.02) weights and N(0, 1) activations drawn on
the device by the seeded generator.  One step = one decode token through all 40 layers
(router, top-k, shared and routed experts, output reduction): one persistent launch per
layer, layers serialised on one stream; the timed steps are captured in a HIP graph and
replayed once between HIP events.  Prints one JSON line.

Other workloads (``--workload``) print their own JSON line with the same keys where they
apply: the tiny fp32 layer, the channel-sparse stack (``--keep``), the MXFP4 stack, and the
linear-expert batch sweep (one line per batch size).

``--gpus N`` with N > 1 exits: this build measures one GPU.
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

METRIC = "MoE-stack decode tokens/s at batch 1 + achieved HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = {
    "b1": ["expert_b1.hip", "layer_common.h", "device_common.h"],
    "cs": ["channel_sparse.hip", "layer_common.h", "device_common.h"],
    "linear": ["linear_mfma.hip", "linear_gemv.hip", "grouped_tn.hip", "route.hip",
               "layer_common.h", "device_common.h"],
}
BYTES_PER_ELEM = {"f32": 4.0, "bf16": 2.0, "mxfp4": 0.5 + 1.0 / 32.0}


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "routed_expert_ffn_route_amd", "csrc", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def layer_weight_bytes(wl, keep=None, n_read=None) -> float:
    """Algorithmic weight bytes one token (or one batch step) reads in one layer: the router,
    the routed experts (k of them; n_read for a batch: the touched ones) and the shared
    experts, 3 matrices of H x I each (linear experts: one matrix, no router).  With a keep
    count (channel-sparse layer): every gate row, the kept up and down rows, the down-norm
    entries of the candidates."""
    be = BYTES_PER_ELEM[wl.expert_dtype]
    bs = BYTES_PER_ELEM.get(wl.shared_dtype, 0.0)
    br = BYTES_PER_ELEM.get(wl.router_dtype, 0.0)
    n = wl.k if n_read is None else n_read
    if wl.kind == "linear":
        return n * wl.H * wl.I * be
    if keep is None:
        routed = n * 3 * wl.H * wl.I * be
    else:
        routed = wl.k * wl.I * wl.H * be + 2 * keep * wl.H * be + 4 * wl.k * wl.I
    return routed + wl.n_shared * 3 * wl.H * wl.I_shared * bs + wl.E * wl.H * br


def traffic_from_profiles(name: str, khash: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled
    by a copy kernel's readings), if they were taken on this kernel source: the last line of
    profiles/traffic_<name>.txt is the JSON record."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = [ln for ln in f if ln.startswith("{")]
    if not recs:
        return None
    d = json.loads(recs[-1])
    if d.get("kernel_hash") != khash:
        return None
    return d.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, sample_layers: int, token: int = 0, keep=None):
    """The oracle, as written, on the host cores: one token through `sample_layers` layers
    (weight generation excluded from the timing).  Returns the record and the outputs."""
    from synth import tensors as T
    from oracle import moe_oracle as O
    total = 0.0
    outs = []
    for layer in range(sample_layers):
        Wr = T.router(wl, layer)
        x = T.x(wl, token, layer, 0)
        ids, w = O.route(O.router_logits(x, Wr), wl.k)
        experts = {int(e): T.expert(wl, layer, int(e)) for e in ids[0]}
        shared = [T.shared(wl, layer, s) for s in range(wl.n_shared)]
        t0 = time.perf_counter()
        if keep is None:
            y, _, _ = O.moe_layer_token(x, Wr, lambda e: experts[e], wl.k, shared)
        else:
            _, y = O.channel_select_token(x, ids[0], w[0], lambda e: experts[e],
                                          lambda e: O.down_norms(experts[e][2]), keep, shared)
        total += time.perf_counter() - t0
        outs.append(y)
    rec = {"value": (sample_layers / wl.layers) / total, "unit": "tokens/s",
           "cores": blas_threads(), "kind": "oracle",
           "sample": f"token {token} through layers 0..{sample_layers - 1} of {wl.layers} "
                     f"(fp64 numpy oracle, weight generation excluded): {total:.2f} s of CPU "
                     f"time, scaled to a full {wl.layers}-layer token"}
    return rec, outs


def timed(fn, steps, graph_ok=True):
    """Capture `steps` calls of fn(t) in a HIP graph (or run eagerly), time one replay with
    HIP events on the launching stream.  Returns (gpu ms, wall ms)."""
    import torch
    graph = None
    if graph_ok:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for t in range(steps):
                fn(t)
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    if graph is not None:
        graph.replay()
    else:
        for t in range(steps):
            fn(t)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end), (time.perf_counter() - w0) * 1e3


def run_stack(args, wl, keep=None):
    """Batch-1 decode through a stack of layers (dense or channel-sparse)."""
    import numpy as np
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    ntok = min(wl.tokens, max(args.steps, 1))
    t_gen = time.perf_counter()
    layers, xs, ys, kepts = [], [], [], []
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    for l in range(wl.layers):
        layers.append(M.Layer(desc, T.device_layer(wl, l)))
        xs.append(T.device_x(wl, list(range(ntok)), l))
        ys.append(torch.empty_like(xs[-1]))
        if keep is not None:
            kepts.append(torch.empty((ntok, max(keep, 1)), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    print(f"# {wl.name}: generated {wl.layers} layers in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    def step(t):
        tt = t % ntok
        for l in range(wl.layers):
            if keep is None:
                layers[l].forward(xs[l][tt:tt + 1], ys[l][tt:tt + 1], B=1)
            else:
                layers[l].channel_select(xs[l][tt:tt + 1], keep, kepts[l][tt],
                                         y=ys[l][tt:tt + 1])

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    for L in layers:
        assert L.check() == 0, "device error word set"
    K = args.steps
    gpu_ms, wall_ms = timed(step, K, graph_ok=not args.eager)
    for L in layers:
        assert L.check() == 0, "device error word set"
    launches = K * wl.layers
    per_launch_s = gpu_ms / 1e3 / launches
    bytes_layer = layer_weight_bytes(wl, keep=keep)
    achieved = bytes_layer / per_launch_s / 1e9
    kind = "b1" if keep is None else "cs"
    khash = kernel_hash(kind)
    name = f"{kind}_layer_{wl.name}" + ("" if keep is None else f"_keep{keep}")
    out = {
        "metric": METRIC,
        "value": round(K / (gpu_ms / 1e3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "inter": wl.I, "shared": wl.n_shared,
                   "weights": wl.expert_dtype, "batch": 1, "keep": keep,
                   "graph": not args.eager},
        "hbm_gb_s": round(achieved, 1),
        "hbm_pct_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall_ms / K, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(name, khash),
                     "kernel": f"{kind}_kernel (one launch per layer)",
                     "bytes_per_launch": bytes_layer,
                     "us_per_launch": round(per_launch_s * 1e6, 3), "kernel_hash": khash},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cb, outs = cpu_baseline(wl, min(args.cpu_layers, wl.layers), token=0, keep=keep)
        worst = 0.0
        for l, y_ref in enumerate(outs):
            y = ys[l][0].cpu().numpy().astype(np.float64)
            worst = max(worst, float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref))))
        cb["token0_max_rel_err_vs_oracle"] = worst
        out["cpu_baseline"] = cb
    return out


def run_batched_stack(args, wl, B):
    """Batched decode (B tokens per step) through the SwiGLU stack: per layer, routing, the
    touched-expert union and the batched expert kernels; each touched expert is read once
    per step for all its tokens."""
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    nb = max(1, min(wl.tokens // B, max(args.steps, 1)))
    t_gen = time.perf_counter()
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=B)
    layers, xs, ys = [], [], []
    for l in range(wl.layers):
        layers.append(M.Layer(desc, T.device_layer(wl, l)))
        xs.append(T.device_x(wl, list(range(nb * B)), l))
        ys.append(torch.empty_like(xs[-1]))
    torch.cuda.synchronize()
    print(f"# {wl.name}: generated {wl.layers} layers in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    # touched experts of every (layer, batch) for the byte figure (untimed)
    ids = torch.empty((B, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, wl.k), dtype=torch.float32, device="cuda")
    nt_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_dev = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    o_dev = torch.empty(wl.E + 1, dtype=torch.int32, device="cuda")
    s_dev = torch.empty(B * wl.k, dtype=torch.int32, device="cuda")
    touched = {}
    for l in range(wl.layers):
        for i in range(nb):
            layers[l].route(x=xs[l][i * B:(i + 1) * B], ids=ids, w=w)
            M.union_experts(ids, wl.E, nt_dev, t_dev, o_dev, s_dev)
            touched[(l, i)] = int(nt_dev.item())

    def step(t):
        i = t % nb
        for l in range(wl.layers):
            layers[l].forward(xs[l][i * B:(i + 1) * B], ys[l][i * B:(i + 1) * B], B=B)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    for L in layers:
        assert L.check() == 0, "device error word set"
    K = args.steps
    gpu_ms, wall_ms = timed(step, K, graph_ok=not args.eager)
    for L in layers:
        assert L.check() == 0, "device error word set"
    step_bytes = sum(layer_weight_bytes(wl, n_read=touched[(l, t % nb)])
                     for t in range(K) for l in range(wl.layers)) / K
    mean_touched = sum(touched.values()) / len(touched)
    achieved = step_bytes / (gpu_ms / 1e3 / K) / 1e9
    return {
        "metric": "MoE-stack batched decode tokens/s (aggregate over the batch)",
        "value": round(K * B / (gpu_ms / 1e3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "inter": wl.I, "shared": wl.n_shared,
                   "weights": wl.expert_dtype, "batch": B, "graph": not args.eager},
        "mean_touched_experts": round(mean_touched, 2),
        "hbm_gb_s": round(achieved, 1),
        "hbm_pct_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall_ms / K, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "route + union + gate/up + down + combine per layer",
                     "bytes_per_step": step_bytes,
                     "us_per_layer_step": round(gpu_ms * 1e3 / K / wl.layers, 3)},
        "cpu_baseline": None,
    }


def run_linear_sweep(args, wl):
    """The linear-expert batch sweep: per batch, one step = route (given iid logits), union,
    and the MFMA grouped product; each step's touched experts are read once."""
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    batches = [int(b) for b in args.batches.split(",")] if args.batches else list(wl.batches)
    bmax = max(batches)
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, kind=M.LINEAR, router_dtype=None,
                       expert_dtype="bf16", max_batch=bmax)
    L = M.Layer(desc, T.device_layer(wl, 0))
    flush = torch.zeros(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(512 * 2**20 // 64, dtype=torch.float32, device="cuda")

    def evict(t):
        # evict the previous step's experts from the 256 MB MALL and the L2s
        if args.flush == "fill":
            flush.fill_(float(t))  # 512 MB of writes (their write-back can overlap the step)
        else:
            sink.copy_(flush.view(-1, 16)[:, 0])  # one 4-byte read per 64-byte piece: 512 MB
                                                  # of lines read, 32 MB written
    lines = []
    for B in batches:
        nsteps = max(2, min(args.steps, 64 if B <= 64 else 16))
        tokens = list(range(B))
        logits = [T.device_logits(wl, tokens, case=3 + s % 4) for s in range(4)]
        x = [T.device_x(wl, tokens, case=3 + s % 4) for s in range(4)]
        ids = torch.empty((B, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((B, wl.k), dtype=torch.float32, device="cuda")
        y = torch.empty((B, wl.I), dtype=torch.float32, device="cuda")
        n_touched = []

        def step(t):
            evict(t)
            L.route(logits_in=logits[t % 4], ids=ids, w=w)
            L.forward(x[t % 4], y, ids=ids, w=w)

        # touched-expert counts of the four routings, for the byte figure (untimed)
        nt_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
        t_dev = torch.empty(wl.E, dtype=torch.int32, device="cuda")
        o_dev = torch.empty(wl.E + 1, dtype=torch.int32, device="cuda")
        s_dev = torch.empty(B * wl.k, dtype=torch.int32, device="cuda")
        for s in range(4):
            L.route(logits_in=logits[s], ids=ids, w=w)
            M.union_experts(ids, wl.E, nt_dev, t_dev, o_dev, s_dev)
            n_touched.append(int(nt_dev.item()))
        for t in range(2):
            step(t)
        torch.cuda.synchronize()
        # time the flush alone and subtract it
        fl_ms, _ = timed(evict, nsteps, graph_ok=not args.eager)
        gpu_ms, _ = timed(step, nsteps, graph_ok=not args.eager)
        assert L.check() == 0
        step_s = (gpu_ms - fl_ms) / 1e3 / nsteps
        touched = sum(n_touched[t % 4] for t in range(nsteps)) / nsteps
        bytes_step = layer_weight_bytes(wl, n_read=touched)
        achieved = bytes_step / step_s / 1e9
        flops = 2.0 * B * wl.k * wl.H * wl.I
        lines.append({
            "metric": "linear-expert batch step time", "workload": wl.name, "batch": B,
            "us_per_step": round(step_s * 1e6, 2), "tokens_per_s": round(B / step_s, 1),
            "touched_experts": touched, "hbm_gb_s": round(achieved, 1),
            "hbm_pct_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
            "tflop_s": round(flops / step_s / 1e12, 2), "steps": nsteps,
            "note": f"MALL flushed before each step (512 MB {args.flush}, timed separately and "
                    "subtracted)", "kernel_hash": kernel_hash("linear")})
    return lines


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode tokens (or steps)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen35_a3b_bf16")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0: workload's)")
    ap.add_argument("--keep", type=int, default=-1,
                    help="channel-sparse workload: kept channels per token (-1: first of the "
                         "workload's keep counts)")
    ap.add_argument("--flush", choices=["read", "fill"], default="read",
                    help="linear sweep: how the MALL is flushed between steps (a strided read "
                         "of 512 MB, or a 512 MB fill)")
    ap.add_argument("--batches", default="", help="linear sweep: comma-separated batch sizes")
    ap.add_argument("--batch", type=int, default=1,
                    help="SwiGLU stacks: tokens per step (B > 1 runs the batched layer)")
    ap.add_argument("--eager", action="store_true", help="launch without a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=40, help="layers in the oracle sample")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB ten times (the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from synth import tensors as T
    from synth.workloads import WORKLOADS
    torch.cuda.set_device(0)
    if args.copy_calibrate:
        n = args.copy_calibrate * 2**20 // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibrate_bytes_each_way": n * 4, "copies": 10}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.layers:
        wl = T.reduced(wl, layers=args.layers)
    if wl.kind == "linear":
        for line in run_linear_sweep(args, wl):
            print(json.dumps(line), flush=True)
        return
    if args.batch > 1:
        print(json.dumps(run_batched_stack(args, wl, args.batch)), flush=True)
        return
    keep = None
    if wl.keep_fracs:
        keep = args.keep if args.keep >= 0 else wl.keep_counts()[0]
    print(json.dumps(run_stack(args, wl, keep)), flush=True)


if __name__ == "__main__":
    main()
