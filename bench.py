#!/usr/bin/env python3
"""MoE-stack decode benchmark on one MI355X: tokens/s at batch 1 and achieved HBM GB/s.

Workload (default): the 40-layer bf16 stack shaped like Qwen3.5-35B-A3B -- H=2048, E=256
routed experts, top-8 with softmax over the selected logits, one always-on shared expert,
expert width I=768 -- with synthetic N(0, 0.02) weights and N(0, 1) activations drawn on
the device by the seeded generator.  One step = one decode token through all 40 layers
(router, top-k, shared and routed experts, output reduction), one persistent launch per
layer, layers serialised on one stream; the timed steps are captured in a HIP graph and
replayed once between HIP events.

Prints one JSON line (see the keys below).  ``--gpus N`` with N > 1 exits: this build runs
on one GPU.
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
DOMINANT_SOURCES = ["routed_expert_ffn_route_amd/csrc/expert_b1.hip",
                    "routed_expert_ffn_route_amd/csrc/device_common.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def layer_weight_bytes(wl) -> int:
    """Algorithmic weight bytes one token reads in one layer: router, k routed experts,
    shared experts (3 matrices of H x I each)."""
    be = {"f32": 4, "bf16": 2}[wl.expert_dtype]
    bs = {"f32": 4, "bf16": 2}.get(wl.shared_dtype, 0)
    br = {"f32": 4, "bf16": 2}.get(wl.router_dtype, 0)
    return (wl.k * 3 * wl.H * wl.I * be + wl.n_shared * 3 * wl.H * wl.I_shared * bs
            + wl.E * wl.H * br)


def traffic_from_profiles(khash: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_b1_layer_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_hash") != khash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, sample_layers: int, token: int = 0):
    """The oracle, as written, on the host cores: one token through `sample_layers` layers."""
    import numpy as np
    from synth import tensors as T
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    total = 0.0
    outs = []
    for layer in range(sample_layers):
        Wr = T.router(wl, layer)
        x = T.x(wl, token, layer, 0)
        logits = O.router_logits(x, Wr)[0]
        ids, _ = O.route(logits[None, :], wl.k)
        experts = {int(e): T.expert(wl, layer, int(e)) for e in ids[0]}
        shared = [T.shared(wl, layer, s) for s in range(wl.n_shared)]
        t0 = time.perf_counter()
        y, _, _ = O.moe_layer_token(x, Wr, lambda e: experts[e], wl.k, shared)
        total += time.perf_counter() - t0
        outs.append(y)
    tokens_per_s = (sample_layers / wl.layers) / total
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"token {token} through layers 0..{sample_layers - 1} of {wl.layers} "
                      f"(fp64 numpy oracle; weight generation excluded); "
                      f"{total:.2f} s of CPU time, scaled to a full {wl.layers}-layer token"}, outs


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode tokens")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen35_a3b_bf16")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0: workload's)")
    ap.add_argument("--eager", action="store_true", help="launch without a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=40, help="layers in the oracle sample")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    from synth.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.layers:
        wl = T.reduced(wl, layers=args.layers)
    assert wl.kind == "swiglu" and wl.expert_dtype in ("f32", "bf16"), "batch-1 bf16/f32 stacks"
    torch.cuda.set_device(0)
    ntok = min(wl.tokens, max(args.steps, 1))

    t_gen = time.perf_counter()
    layers, xs, ys = [], [], []
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    for l in range(wl.layers):
        layers.append(M.Layer(desc, T.device_layer(wl, l)))
        xs.append(T.device_x(wl, list(range(ntok)), l))
        ys.append(torch.empty_like(xs[-1]))
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"# generated {wl.layers} layers ({layer_weight_bytes(wl)} B/token-layer read) "
          f"in {t_gen:.1f} s", file=sys.stderr, flush=True)

    def step(t):
        tt = t % ntok
        for l in range(wl.layers):
            layers[l].forward(xs[l][tt:tt + 1], ys[l][tt:tt + 1], B=1)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    for L in layers:
        assert L.check() == 0

    K = args.steps
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for t in range(K):
                step(t)
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
        for t in range(K):
            step(t)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = start.elapsed_time(end)
    for L in layers:
        assert L.check() == 0, "device error word set"

    launches = K * wl.layers
    per_launch_s = gpu_ms / 1e3 / launches
    bytes_layer = layer_weight_bytes(wl)
    tokens_per_s = K / (gpu_ms / 1e3)
    achieved = bytes_layer / per_launch_s / 1e9
    khash = kernel_hash()
    traffic = traffic_from_profiles(khash, wl.name)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
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
        "config": {"workload": wl.name, "layers": wl.layers, "hidden": wl.H,
                   "experts": wl.E, "top_k": wl.k, "inter": wl.I, "shared": wl.n_shared,
                   "weights": wl.expert_dtype, "batch": 1, "graph": graph is not None},
        "hbm_gb_s": round(achieved, 1),
        "hbm_pct_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "b1_kernel (one launch per layer)",
                     "bytes_per_launch": bytes_layer,
                     "us_per_launch": round(per_launch_s * 1e6, 3),
                     "kernel_hash": khash},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import numpy as np
        cb, outs = cpu_baseline(wl, min(args.cpu_layers, wl.layers), token=0)
        # the timed outputs of token 0 against the oracle (information only)
        worst = 0.0
        for l, y_ref in enumerate(outs):
            y = ys[l][0].cpu().numpy().astype(np.float64)
            worst = max(worst, float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref))))
        cb["token0_max_rel_err_vs_oracle"] = worst
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
