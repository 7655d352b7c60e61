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


def layer_weight_bytes(wl, keep=None, n_read=None, sketch=False, recover=False) -> float:
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
    elif sketch:
        # the sketch of every candidate's gate and up rows (2-bit codes + an FP16 scale per
        # 128-block), then the kept channels' full gate, up and down rows, and the norms
        routed = (wl.k * wl.I * 2 * (wl.H // 128) * (32 + 2) + 3 * keep * wl.H * be +
                  4 * wl.k * wl.I)
        if recover:  # (reader) b_j of every dropped candidate (32 FP16) and U (H x 32 fp32)
            routed += (wl.k * wl.I - keep) * 32 * 2 + wl.H * 32 * 4
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Host threads this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, sample_layers: int, token: int = 0, keep=None):
    """The C++ oracle (oracle/cpp/moe_oracle.cpp: plain loops, double accumulation), as
    written, on the host: one token through `sample_layers` layers, timed at 1 thread and at
    every host thread of this process (independent outputs split over threads).  Host weight
    generation is outside the timing.  Returns the record and the layer outputs."""
    from synth import tensors as T
    from oracle import cpp_oracle as C
    nthr = host_threads()
    totals = {1: 0.0, nthr: 0.0}
    outs = []
    for layer in range(sample_layers):
        Wr = T.router(wl, layer)
        x = T.x(wl, token, layer, 0)
        ids, w = C.route(C.router_logits(x, Wr), wl.k)
        experts = {int(e): T.expert(wl, layer, int(e)) for e in ids[0]}
        shared = [T.shared(wl, layer, s) for s in range(wl.n_shared)]
        dn = {}
        if keep is not None:
            dn = {e: C.down_norms(experts[e][2]) for e in experts}
        for th in totals:
            C.set_threads(th)
            t0 = time.perf_counter()
            if keep is None:
                y, _, _ = C.moe_layer_token(x, Wr, lambda e: experts[e], wl.k, shared)
            else:
                _, y = C.channel_select_token(x, ids[0], w[0], lambda e: experts[e],
                                              dn.__getitem__, keep, shared)
            totals[th] += time.perf_counter() - t0
        C.set_threads(1)
        outs.append(y)
    scale = sample_layers / wl.layers
    rec = {"value": round(scale / totals[nthr], 4), "unit": "tokens/s", "cores": nthr,
           "kind": "oracle", "value_1_thread": round(scale / totals[1], 4),
           "cpu_model": cpu_model(),
           "sample": f"token {token} through layers 0..{sample_layers - 1} of {wl.layers} (C++ "
                     f"fp64 oracle, host weight generation excluded): {totals[1]:.2f} s wall "
                     f"at 1 thread, {totals[nthr]:.2f} s at {nthr} threads, scaled to a full "
                     f"{wl.layers}-layer token"}
    return rec, outs


_PROBE = None


def probe_lib():
    global _PROBE
    if _PROBE is None:
        import ctypes
        path = os.path.join(ROOT, "routed_expert_ffn_route_amd", "libmoe_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python routed_expert_ffn_route_amd/build.py`")
        L = ctypes.CDLL(path)
        L.probe_stream_read.restype = ctypes.c_int
        L.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.probe_empty.restype = ctypes.c_int
        L.probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _PROBE = L
    return _PROBE


def stream_probe(gib: int = 4, reps: int = 5) -> float:
    """Achieved HBM read bandwidth (GB/s): a read-only stream over `gib` GiB (16 times the
    256 MB MALL, so nothing is served from it) with non-temporal 16-byte loads (each wave's
    load one contiguous KiB), timed over `reps` launches with HIP events on the launching
    stream; the best of four grid sizes (1024 to 8192 workgroups of 256 threads)."""
    import torch
    L = probe_lib()
    nbytes = gib * 2**30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            assert L.probe_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), st) == 0
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            assert L.probe_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), st) == 0
        end.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (start.elapsed_time(end) / 1e3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def launch_floor(workgroups: int, threads: int, nodes: int = 40, reps: int = 50) -> float:
    """Microseconds per launch of an empty kernel with the layer kernel's geometry, `nodes`
    launches captured in one HIP graph and replayed `reps` times: the per-layer floor that
    dispatch alone sets."""
    import torch
    L = probe_lib()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(nodes):
                assert L.probe_empty(workgroups, threads,
                                     torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (reps * nodes)


def platform_figures(achieved_gbs: float, workgroups: int, threads: int) -> dict:
    """The probe bandwidth, the achieved rate as a share of it, and the launch floor."""
    probe = stream_probe()
    return {"probe_gb_s": round(probe, 1), "pct_of_probe": round(100 * achieved_gbs / probe, 2),
            "launch_floor_us": round(launch_floor(workgroups, threads), 3)}


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
    """Batch-1 decode through a stack of layers (dense, channel-sparse, or channel-sparse with
    the ternary-sketch screen)."""
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
        if args.sketch:
            layers[-1].build_sketch(torch.from_numpy(T.rotation_signs(wl, l)).cuda())
        if args.recover:
            layers[-1].build_recovery(recovery_basis_device(layers[-1].tensors["down_t"], wl))
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
                                         y=ys[l][tt:tt + 1], sketch=args.sketch,
                                         reader=args.recover, mode=1 if args.sketch else 0)

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
    bytes_layer = layer_weight_bytes(wl, keep=keep, sketch=args.sketch, recover=args.recover)
    achieved = bytes_layer / per_launch_s / 1e9
    kind = "b1" if keep is None else "cs"
    khash = kernel_hash(kind)
    name = f"{kind}_layer_{wl.name}" + ("" if keep is None else f"_keep{keep}") + \
        ("_sketch" if args.sketch else "")
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
                   "screen": ("ternary sketch, eq. 1, rank-32 recovery (eq. 2)"
                              if args.recover else
                              "ternary sketch, eq. 1" if args.sketch else
                              "exact gates" if keep is not None else None),
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
    wgs, thr = layers[0].geometry()
    out.update(platform_figures(achieved, wgs, thr))
    if not args.no_cpu_baseline and not args.sketch:
        cb, outs = cpu_baseline(wl, min(args.cpu_layers, wl.layers), token=0, keep=keep)
        worst = 0.0
        for l, y_ref in enumerate(outs):
            y = ys[l][0].cpu().numpy().astype(np.float64)
            worst = max(worst, float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref))))
        cb["token0_max_rel_err_vs_oracle"] = worst
        out["cpu_baseline"] = cb
    return out


def recovery_basis_device(down_t, wl, rank=32):
    """U [H][rank] for a layer (load-time preparation, outside any timed region): the top
    eigenvectors of sum_j d_j d_j^T over its stacked down columns, by torch on the GPU."""
    import torch
    D = down_t.view(torch.bfloat16).reshape(-1, wl.H) if down_t.dtype != torch.float32 else \
        down_t.reshape(-1, wl.H)
    G = torch.zeros((wl.H, wl.H), dtype=torch.float64, device=down_t.device)
    for i in range(0, D.shape[0], 16384):
        blk = D[i:i + 16384].to(torch.float32)
        G += (blk.T @ blk).to(torch.float64)
    vals, vecs = torch.linalg.eigh(G)
    return vecs[:, -rank:].flip(1).to(torch.float32).contiguous()


def run_threshold(args, wl):
    """The threshold keep rule through the 40-layer stack ("Background: channels and keep
    rules" and the calibration discussion of the reader review).  Per layer, tau is
    calibrated so that a fraction `--threshold` of the pooled exact scores of 16 calibration
    tokens is at or above it (the scores read back with moe_layer_scores); then held-out
    tokens are timed, and the per-token kept fraction is reported for them and for a shifted
    set (the same tokens with x scaled by 0.8: smaller activations, smaller scores -- a
    synthetic stand-in for the review's chat-to-benchmark shift)."""
    import numpy as np
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    frac = args.threshold
    n = wl.k * wl.I
    ncal = 16
    ntok = min(wl.tokens - ncal, max(args.steps, 1))
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    layers, xs, ys, taus = [], [], [], []
    kept = torch.empty(n, dtype=torch.int32, device="cuda")
    sc = torch.empty(n, dtype=torch.float32, device="cuda")
    K0 = int(np.floor(frac * n + 0.5))
    for l in range(wl.layers):
        L = M.Layer(desc, T.device_layer(wl, l))
        layers.append(L)
        xcal = T.device_x(wl, list(range(ncal)), l)
        pooled = []
        for t in range(ncal):  # calibration tokens 0 .. 15
            L.channel_select(xcal[t:t + 1], K0, kept, mode=1)
            L.scores(sc)
            pooled.append(sc.cpu().numpy().astype(np.float64))
        pooled = np.sort(np.concatenate(pooled))[::-1]
        taus.append(float(pooled[int(np.floor(frac * pooled.size + 0.5)) - 1]))
        xs.append(T.device_x(wl, list(range(ncal, ncal + ntok)), l))  # held-out tokens
        ys.append(torch.empty_like(xs[-1]))
    torch.cuda.synchronize()
    counts = torch.zeros((2, ntok, wl.layers), dtype=torch.int32, device="cuda")
    kepts = torch.empty((wl.layers, n), dtype=torch.int32, device="cuda")

    def step_on(xsrc, which):
        def step(t):
            tt = t % ntok
            for l in range(wl.layers):
                layers[l].channel_select_threshold(xsrc[l][tt:tt + 1], taus[l], kepts[l],
                                                   counts[which, tt, l:l + 1],
                                                   y=ys[l][tt:tt + 1], mode=1)
        return step

    step = step_on(xs, 0)
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    K = ntok
    gpu_ms, wall_ms = timed(step, K, graph_ok=not args.eager)
    for L in layers:
        assert L.check() == 0, "device error word set"
    shifted = [0.8 * x for x in xs]
    sstep = step_on(shifted, 1)
    for t in range(ntok):
        sstep(t)
    torch.cuda.synchronize()
    for L in layers:
        assert L.check() == 0, "device error word set"
    c = counts.cpu().numpy().astype(np.float64) / n

    def dist(a):
        a = a.ravel()
        return {"mean": round(float(a.mean()), 4), "min": round(float(a.min()), 4),
                "p5": round(float(np.percentile(a, 5)), 4),
                "p50": round(float(np.percentile(a, 50)), 4),
                "p95": round(float(np.percentile(a, 95)), 4), "max": round(float(a.max()), 4)}

    mean_kept = float(c[0].mean()) * n
    bytes_layer = layer_weight_bytes(wl, keep=mean_kept)
    per_launch_s = gpu_ms / 1e3 / (K * wl.layers)
    achieved = bytes_layer / per_launch_s / 1e9
    return {
        "metric": METRIC, "value": round(K / (gpu_ms / 1e3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(gpu_ms / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "batch": 1,
                   "keep_rule": "threshold", "calibrated_fraction": frac,
                   "calibration_tokens": ncal, "score": "router-weighted, exact gates",
                   "graph": not args.eager},
        "kept_fraction_held_out": dist(c[0]),
        "kept_fraction_shifted_x0.8": dist(c[1]),
        "tau_per_layer_first4": [round(t, 6) for t in taus[:4]],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "cs_kernel (one launch per layer)",
                     "bytes_per_launch": bytes_layer,
                     "us_per_launch": round(per_launch_s * 1e6, 3),
                     "kernel_hash": kernel_hash("cs")},
        "cpu_baseline": None,
    }


PHASES = {
    "b1": {0: "start", 1: "router rows published", 2: "shared experts streamed",
           3: "routing known (top-k + softmax)", 4: "routed stream done",
           5: "partial output summed in LDS", 6: "shared rows prefetched (wave 4)",
           7: "reducer: every thread's partials seen", 8: "top-k: wave 0 keys sorted in runs",
           9: "top-k: wave 0 top of its keys",
           10: "top-k: wave 0 keys polled", 11: "top-k: ranked", 12: "router rows computed",
           13: "partial output published", 14: "reducer: all partials arrived",
           15: "reducer: y written"},
    "cs": {0: "start", 1: "router rows published", 3: "routing known (top-k + softmax)",
           4: "own scores published", 2: "shared experts streamed",
           5: "all scores gathered", 6: "threshold known", 23: "own kept list ready",
           24: "kept rows streamed", 7: "reducer: every thread's partials seen", 8: "top-k: wave 0 keys sorted in runs",
           9: "top-k: wave 0 top of its keys", 10: "top-k: wave 0 keys polled",
           11: "top-k: ranked", 12: "router rows computed", 13: "partial output published",
           14: "reducer: all partials arrived", 15: "reducer: y written",
           16: "gather: scores in (wave 0)", 17: "select: histogram done",
           18: "select: bin found", 19: "select: bin members listed"},
}


def run_timeline(args, wl, keep=None):
    """Phase timeline of the single-launch layer kernel: the library's timeline build records,
    per workgroup, the 100 MHz constant clock at the end of each phase.  The launches of
    `steps` tokens through the stack are captured in one HIP graph (each launch with its own
    stamp rows) and replayed once; per launch, times are taken from the earliest workgroup
    start, then the median over launches of the median and the maximum over workgroups."""
    import numpy as np
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    L = M.use_timeline_library()
    ntok = min(wl.tokens, max(args.steps, 1))
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    layers, xs, ys, kepts = [], [], [], []
    for l in range(wl.layers):
        layers.append(M.Layer(desc, T.device_layer(wl, l)))
        xs.append(T.device_x(wl, list(range(ntok)), l))
        ys.append(torch.empty_like(xs[-1]))
        if keep is not None:
            kepts.append(torch.empty((ntok, max(keep, 1)), dtype=torch.int32, device="cuda"))
        if args.sketch:
            layers[-1].build_sketch(torch.from_numpy(T.rotation_signs(wl, l)).cuda())
    P = layers[0].geometry()[0]
    K = args.steps
    nl = K * wl.layers
    per = 512 * 32
    stamps = torch.zeros(nl * per, dtype=torch.int64, device="cuda")

    def launch(t, l, rec):
        L.moe_debug_set_stamps(ctypes_ptr(stamps, rec * per) if rec is not None else None)
        tt = t % ntok
        if keep is None:
            layers[l].forward(xs[l][tt:tt + 1], ys[l][tt:tt + 1], B=1)
        else:
            layers[l].channel_select(xs[l][tt:tt + 1], keep, kepts[l][tt], y=ys[l][tt:tt + 1],
                                     sketch=args.sketch, mode=1 if args.sketch else 0)

    for t in range(args.warmup):
        for l in range(wl.layers):
            launch(t, l, None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(K):
            for l in range(wl.layers):
                launch(t, l, t * wl.layers + l)
    L.moe_debug_set_stamps(None)
    torch.cuda.synchronize()
    stamps.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for lay in layers:
        assert lay.check() == 0, "device error word set"
    st = stamps.view(nl, 512, 32).cpu().numpy()[:, :P, :].astype(np.int64)
    kind = "b1" if keep is None else "cs"
    names = PHASES[kind]
    rows = []
    t0 = st[:, :, 0].min(axis=1)  # earliest workgroup start per launch
    for i, name in sorted(names.items()):
        med, mx = [], []
        for n in range(nl):
            v = st[n, :, i]
            v = v[v > 0]
            if v.size:
                med.append(np.median(v - t0[n]) * 0.01)
                mx.append(np.max(v - t0[n]) * 0.01)
        if med:
            rows.append({"phase": i, "name": name, "median_us": round(float(np.median(med)), 2),
                         "max_us": round(float(np.median(mx)), 2)})
    # per XCD (workgroup w runs on XCD w % 8): median over launches of the median over the
    # XCD's workgroups, for the end of the stream and the publish
    per_xcd = {}
    for i in (4, 13):
        if i in names:
            vals = []
            for x in range(8):
                med = [np.median(st[n, x::8, i][st[n, x::8, i] > 0] - t0[n]) * 0.01
                       for n in range(nl) if (st[n, x::8, i] > 0).any()]
                vals.append(round(float(np.median(med)), 2) if med else None)
            per_xcd[names[i]] = vals
    # shader clock: s_memtime ticks between the start and the publish of the partial output,
    # over the 100 MHz clock between the same two points
    ticks = (st[:, :, 31] - st[:, :, 30]).astype(np.float64)
    real = (st[:, :, 13] - st[:, :, 0]).astype(np.float64) * 10.0  # ns
    ok = (ticks > 0) & (real > 0)
    clock_ghz = round(float(np.median(ticks[ok] / real[ok])), 3) if ok.any() else None
    st = st[:, :, :30]
    # start of launch n+1 (earliest workgroup) after the last stamp of launch n
    last = st.max(axis=(1, 2))
    gaps = [(t0[n + 1] - last[n]) * 0.01 for n in range(nl - 1)]
    span = [(last[n] - t0[n]) * 0.01 for n in range(nl)]
    return {"timeline": kind, "workload": wl.name, "keep": keep, "launches": nl,
            "workgroups": P, "phases": rows, "per_xcd_median_us": per_xcd,
            "shader_clock_ghz": clock_ghz,
            "first_start_to_last_stamp_us": round(float(np.median(span)), 2),
            "last_stamp_to_next_start_us": round(float(np.median(gaps)), 2) if gaps else None,
            "note": "100 MHz constant clock (10 ns); median over launches of the per-launch "
                    "median / max over workgroups, from the earliest workgroup start"}


def ctypes_ptr(t, offset_elems=0):
    import ctypes
    return ctypes.c_void_p(t.data_ptr() + offset_elems * t.element_size())


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
    wgs, thr = layers[0].geometry()
    plat = platform_figures(achieved, wgs, thr)
    return {**plat, 
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


def run_batch_select(args, wl, B, keep_tok):
    """Batch-wide channel selection through the channel-sparse stack (the reader review's
    "Limits": one kept set for the whole batch).  Per layer and step of B tokens: routing, the
    touched-expert union, the batch scores from every touched gate row, the selection of
    keep = B * keep_tok channels, the kept channels' activations and down products for the
    tokens routed to them, the shared experts for every token."""
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    nb = max(1, min(wl.tokens // B, max(args.steps, 1)))
    keep = B * keep_tok
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=B)
    layers, xs, ys = [], [], []
    for l in range(wl.layers):
        layers.append(M.Layer(desc, T.device_layer(wl, l)))
        xs.append(T.device_x(wl, list(range(nb * B)), l))
        ys.append(torch.empty_like(xs[-1]))
    kept = torch.empty(keep, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
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
    torch.cuda.synchronize()

    def step(t):
        i = t % nb
        for l in range(wl.layers):
            layers[l].channel_select_batch(xs[l][i * B:(i + 1) * B], keep, kept,
                                           ys[l][i * B:(i + 1) * B], kept_count=cnt)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    for L in layers:
        assert L.check() == 0, "device error word set"
    K = args.steps
    gpu_ms, wall_ms = timed(step, K, graph_ok=not args.eager)
    for L in layers:
        assert L.check() == 0, "device error word set"
    be = BYTES_PER_ELEM[wl.expert_dtype]
    bs = BYTES_PER_ELEM.get(wl.shared_dtype, 0.0)
    br = BYTES_PER_ELEM.get(wl.router_dtype, 0.0)

    def layer_bytes(nt):
        # every touched gate row and its norm, the kept up and down rows, shared, router
        kk = min(keep, nt * wl.I)
        return (nt * wl.I * (wl.H * be + 4) + 2 * kk * wl.H * be +
                wl.n_shared * 3 * wl.H * wl.I_shared * bs + wl.E * wl.H * br)

    step_bytes = sum(layer_bytes(touched[(l, t % nb)])
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
                   "weights": wl.expert_dtype, "batch": B, "keep": keep,
                   "screen": "batch-wide exact gates (summed router-weighted scores)",
                   "graph": not args.eager},
        "mean_touched_experts": round(mean_touched, 2),
        "hbm_gb_s": round(achieved, 1),
        "hbm_pct_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall_ms / K, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "route + union + scores + select + act + down + sum per layer",
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
    gen = None
    if args.torch_inputs:
        # the same shapes and distributions from torch's own device generator (seeded), so
        # that a profiled run launches no kernel of the input generator library
        gen = torch.Generator(device="cuda")
        gen.manual_seed(wl.seed)
        mat = torch.empty((wl.E * wl.I, wl.H), dtype=torch.bfloat16, device="cuda")
        for r0 in range(0, wl.E * wl.I, 8192):
            mat[r0:r0 + 8192].normal_(0.0, wl.sigma_gate, generator=gen)
        L = M.Layer(desc, {"linear": mat})
    else:
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
    probe = stream_probe()
    wgs, thr = L.geometry()
    floor = launch_floor(wgs, thr)
    for B in batches:
        nsteps = max(2, min(args.steps, 64 if B <= 64 else 16))
        tokens = list(range(B))
        if gen is not None:
            logits = [torch.randn((B, wl.E), generator=gen, device="cuda") * wl.sigma_logits
                      for _ in range(4)]
            x = [torch.randn((B, wl.H), generator=gen, device="cuda") * wl.sigma_x
                 for _ in range(4)]
        else:
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
            "probe_gb_s": round(probe, 1), "pct_of_probe": round(100 * achieved / probe, 2),
            "launch_floor_us": round(floor, 3),
            "note": f"MALL flushed before each step (512 MB {args.flush}, timed separately and "
                    "subtracted)", "kernel_hash": kernel_hash("linear")})
    return lines


def run_linear_ek_sweep(args, wl):
    """The batch-1 linearity sub-sweep over (E, k) ("501B of which 23B are switched on",
    section 3[A]: batch-1 time against the expert count and top-k): E = 8, 16, 32, 64 and
    k = 1, 2, 4, 8 linear experts of 8192 x 8192 bf16 (the workload's first E experts), one
    token routed by iid logits, the MALL flushed before each step.  The time should not depend
    on E and should grow linearly in k; the last line fits time = a + b k over all points."""
    import numpy as np
    import torch
    import routed_expert_ffn_route_amd as M
    from synth import tensors as T
    weights = T.device_layer(wl, 0)  # all 64 experts; a layer of E experts reads the first E
    flush = torch.zeros(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(512 * 2**20 // 64, dtype=torch.float32, device="cuda")

    def evict(t):
        sink.copy_(flush.view(-1, 16)[:, 0])

    probe = stream_probe()
    lines, pts = [], []
    nsteps = max(4, min(args.steps, 64))
    for E in (8, 16, 32, 64):
        for k in (1, 2, 4, 8):
            desc = M.make_desc(wl.H, E, k, wl.I, kind=M.LINEAR, router_dtype=None,
                               expert_dtype="bf16", max_batch=1)
            L = M.Layer(desc, weights)
            logits = [T.device_logits(wl, [0], case=3 + s)[:, :E].contiguous()
                      for s in range(4)]
            x = [T.device_x(wl, [0], case=3 + s) for s in range(4)]
            ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
            w = torch.empty((1, k), dtype=torch.float32, device="cuda")
            y = torch.empty((1, wl.I), dtype=torch.float32, device="cuda")

            def step(t):
                evict(t)
                L.route(logits_in=logits[t % 4], ids=ids, w=w)
                L.forward(x[t % 4], y, ids=ids, w=w)

            for t in range(2):
                step(t)
            torch.cuda.synchronize()
            fl_ms, _ = timed(evict, nsteps, graph_ok=not args.eager)
            gpu_ms, _ = timed(step, nsteps, graph_ok=not args.eager)
            assert L.check() == 0
            step_s = (gpu_ms - fl_ms) / 1e3 / nsteps
            nbytes = k * wl.H * wl.I * 2
            pts.append((k, step_s))
            lines.append({
                "metric": "linear-expert batch-1 step time", "workload": wl.name,
                "experts": E, "top_k": k, "us_per_step": round(step_s * 1e6, 2),
                "bytes_per_step": nbytes, "hbm_gb_s": round(nbytes / step_s / 1e9, 1),
                "pct_of_probe": round(100 * nbytes / step_s / 1e9 / probe, 2), "steps": nsteps,
                "note": "MALL flushed before each step (512 MB read, timed separately and "
                        "subtracted)"})
            L.close()
            del L
    ks = np.array([p[0] for p in pts], dtype=np.float64)
    ts = np.array([p[1] for p in pts], dtype=np.float64) * 1e6
    b, a = np.polyfit(ks, ts, 1)
    resid = ts - (a + b * ks)
    per_e = {}
    for (k, t), line in zip(pts, lines):
        per_e.setdefault(k, []).append(t * 1e6)
    lines.append({
        "metric": "linear-expert batch-1 linearity fit", "workload": wl.name,
        "fit": "us = a + b * k over E in (8, 16, 32, 64), k in (1, 2, 4, 8)",
        "a_us": round(float(a), 2), "b_us_per_expert": round(float(b), 2),
        "max_abs_residual_us": round(float(np.max(np.abs(resid))), 2),
        "spread_over_E_us": {str(k): round(max(v) - min(v), 2) for k, v in per_e.items()},
        "bytes_per_expert": wl.H * wl.I * 2, "probe_gb_s": round(probe, 1)})
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
    ap.add_argument("--batch-select", action="store_true",
                    help="sparse workload with --batch B: batch-wide channel selection, "
                         "B * keep channels for the batch (moe_channel_select_batch)")
    ap.add_argument("--sweep-ek", action="store_true",
                    help="linear workload: the batch-1 (E, k) linearity sub-sweep")
    ap.add_argument("--timeline", action="store_true",
                    help="batch-1 stacks: per-phase timeline from the timeline build of the "
                         "library (libmoe_ffn_timeline.so) instead of the throughput line")
    ap.add_argument("--threshold", type=float, default=0.0, metavar="FRAC",
                    help="sparse workload: the threshold keep rule, tau calibrated per layer "
                         "to keep FRAC of the calibration tokens' candidates")
    ap.add_argument("--recover", action="store_true",
                    help="with --sketch: the reader's rank-32 recovery of the dropped channels")
    ap.add_argument("--sketch", action="store_true",
                    help="channel-sparse workload: score channels from the ternary sketch "
                         "(moe_channel_select_sketch, eq.-1 scores) instead of exact gates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--torch-inputs", action="store_true",
                    help="linear sweep: weights, x and logits from torch's device generator "
                         "(no input-generator kernels in the run)")
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
        run = run_linear_ek_sweep if args.sweep_ek else run_linear_sweep
        for line in run(args, wl):
            print(json.dumps(line), flush=True)
        return
    keep = None
    if wl.keep_fracs:
        keep = args.keep if args.keep >= 0 else wl.keep_counts()[0]
    if args.batch > 1 and keep is not None and args.batch_select:
        print(json.dumps(run_batch_select(args, wl, args.batch, keep)), flush=True)
        return
    if args.batch > 1:
        print(json.dumps(run_batched_stack(args, wl, args.batch)), flush=True)
        return
    if args.threshold > 0:
        if not wl.keep_fracs:
            raise SystemExit("--threshold needs the channel-sparse workload")
        print(json.dumps(run_threshold(args, wl)), flush=True)
        return
    if args.timeline:
        print(json.dumps(run_timeline(args, wl, keep)), flush=True)
        return
    print(json.dumps(run_stack(args, wl, keep)), flush=True)


if __name__ == "__main__":
    main()
