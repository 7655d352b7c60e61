"""GPU parity of the batched SwiGLU layer (B > 1: routing, touched-expert union, MFMA
gate/up, down partials, per-token combine) against the oracle, token by token."""
import numpy as np
import pytest

from gpu_common import (HostLayer, TOL_BF16, TOL_MXFP4, corrupt, cuda_ok, pick_attempt,
                        rel_err, used_choices as _used)
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _layer(wl, max_batch, layer=0):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=max_batch)
    return M.Layer(desc, T.device_layer(wl, layer))


def _batch(wl, hl, B, case=0, layer=0):
    """B margin-checked tokens: redraw attempts and the host copies of x."""
    attempts, xs = [], []
    for b in range(B):
        a, x = pick_attempt(wl, b, layer, case=case, host_router=hl.router)
        attempts.append(a)
        xs.append(np.asarray(x, dtype=np.float32).reshape(-1))
    return attempts, np.stack(xs)


def _oracle(wl, hl, X, tokens=None):
    tokens = range(len(X)) if tokens is None else tokens
    ys, ids, ws = {}, {}, {}
    for b in tokens:
        y, i, w = O.moe_layer_token(X[b], hl.router, hl.expert, wl.k, hl.shared)
        ys[b], ids[b], ws[b] = y, i, w
    return ys, ids, ws


def _tol(wl):
    return TOL_MXFP4 if wl.expert_dtype == "mxfp4" else TOL_BF16


# Shapes with ragged tails everywhere: H not a multiple of the 128-wide MXFP4 step (2080),
# I and I_s not multiples of the 256-channel gate/up block or of 16-row tiles, buckets above
# the 64-token pass (E=4, B=200; the shared experts at B=70), and more pairs per expert
# than one down pass takes.
SMALL = [
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=151, H=352, E=37, k=5, I=72, n_shared=1,
              I_shared=56, layers=1),
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=152, H=2080, E=16, k=4, I=296, n_shared=2,
              I_shared=96, layers=1),
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=153, H=256, E=4, k=2, I=40, n_shared=0,
              I_shared=0, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=154, H=1024, E=40, k=4, I=96, n_shared=2,
              I_shared=64, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=155, H=7168, E=64, k=16, I=40, n_shared=1,
              I_shared=24, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=156, H=2080, E=17, k=3, I=200, n_shared=0,
              I_shared=0, layers=1),
    # MXFP4 buckets above 32 tokens (passes of 32), H a multiple of 512 (pipelined steps with
    # the paired scale loads) and not (masked steps only); shared bf16 expert above 64
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=157, H=1024, E=4, k=2, I=72, n_shared=1,
              I_shared=40, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=158, H=2080, E=3, k=2, I=48, n_shared=0,
              I_shared=0, layers=1),
]
BATCHES = {151: (2, 7, 40), 152: (70,), 153: (200,), 154: (3, 16), 155: (16,), 156: (9,),
           157: (70,), 158: (50,)}
CASES = [(wl, B) for wl in SMALL for B in BATCHES[wl.wid]]


@pytest.mark.parametrize("wl,B", CASES,
                         ids=[f"H{w.H}E{w.E}k{w.k}I{w.I}s{w.n_shared}{w.expert_dtype}-B{B}"
                              for w, B in CASES])
def test_batched_given_routing(wl, B):
    import torch
    L = _layer(wl, max_batch=B)
    hl = HostLayer(wl)
    attempts, X = _batch(wl, hl, B)
    ys, ids, ws = _oracle(wl, hl, X)
    x = T.device_x(wl, list(range(B)), attempts=attempts)
    assert np.array_equal(x.cpu().numpy(), X)
    ids_t = torch.from_numpy(np.stack([ids[b] for b in range(B)]).astype(np.int32)).cuda()
    w_t = torch.from_numpy(np.stack([ws[b] for b in range(B)]).astype(np.float32)).cuda()
    y = torch.full((B, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    L.forward(x, y, ids=ids_t, w=w_t)
    assert L.check() == 0
    yc = y.cpu().numpy()
    worst = max(rel_err(yc[b], ys[b]) for b in range(B))
    print(f"B={B}: worst max|dy|/||y||inf = {worst:.3e}")
    assert worst <= _tol(wl)


@pytest.mark.parametrize("wl", [SMALL[0], SMALL[3]], ids=lambda w: w.expert_dtype)
def test_batched_internal_routing_matches_b1_and_oracle(wl):
    """Routing inside the call; every token also equals the batch-1 kernel's output."""
    import torch
    B = 12
    L = _layer(wl, max_batch=B)
    hl = HostLayer(wl)
    attempts, X = _batch(wl, hl, B, case=1)
    ys, _, _ = _oracle(wl, hl, X)
    x = T.device_x(wl, list(range(B)), attempts=attempts, case=1)
    y = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
    L.forward(x, y)
    assert L.check() == 0
    y1 = torch.empty((1, wl.H), dtype=torch.float32, device="cuda")
    for b in range(B):
        assert rel_err(y[b].cpu().numpy(), ys[b]) <= _tol(wl)
        L.forward(x[b:b + 1], y1, B=1)
        assert rel_err(y[b].cpu().numpy(), y1[0].cpu().numpy()) <= _tol(wl)


def test_batched_deterministic():
    import torch
    wl = SMALL[1]
    B = 70
    L = _layer(wl, max_batch=B)
    hl = HostLayer(wl)
    attempts, _ = _batch(wl, hl, B, case=2)
    x = T.device_x(wl, list(range(B)), attempts=attempts, case=2)
    y1 = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    L.forward(x, y1)
    L.forward(x, y2)
    assert L.check() == 0
    assert torch.equal(y1, y2)


def test_batched_one_token_batch_of_smaller_B():
    """A layer sized for B=40 called with B=2 and B=40 in turn (workspace reuse)."""
    import torch
    wl = SMALL[0]
    L = _layer(wl, max_batch=40)
    hl = HostLayer(wl)
    for B in (40, 2, 40):
        attempts, X = _batch(wl, hl, B, case=3)
        ys, _, _ = _oracle(wl, hl, X)
        x = T.device_x(wl, list(range(B)), attempts=attempts, case=3)
        y = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
        L.forward(x, y)
        assert L.check() == 0
        assert max(rel_err(y[b].cpu().numpy(), ys[b]) for b in range(B)) <= TOL_BF16


@pytest.mark.parametrize("name,B,sample", [("mxfp4_e896_k16", 16, (0, 7, 15)),
                                           ("qwen35_a3b_bf16", 64, (0, 21, 63))])
def test_batched_full_size_sampled(name, B, sample):
    """Full layer shapes (E=896 k=16 MXFP4 with two bf16 shared experts at B=16; the
    E=256 k=8 bf16 stack's layer at B=64), internal routing, sampled tokens vs the oracle."""
    import torch
    wl = WORKLOADS[name]
    L = _layer(wl, max_batch=B)
    hl = HostLayer(wl)
    attempts = [pick_attempt(wl, b, 0, case=4, host_router=hl.router)[0] for b in range(B)]
    x = T.device_x(wl, list(range(B)), attempts=attempts, case=4)
    y = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
    L.forward(x, y)
    assert L.check() == 0
    yc = y.cpu().numpy()
    xc = x.cpu().numpy()
    # the routing step of the batched call, every token of the batch against the oracle
    rid = torch.empty((B, wl.k), dtype=torch.int32, device="cuda")
    rw = torch.empty((B, wl.k), dtype=torch.float32, device="cuda")
    L.routing(rid, rw, B=B)
    ids_ref, w_ref = O.route(O.router_logits(xc, hl.router), wl.k)
    assert np.array_equal(rid.cpu().numpy(), ids_ref)
    assert np.max(np.abs(rw.cpu().numpy() - w_ref)) <= 1e-6
    worst = 0.0
    for b in sample:
        y_ref, _, _ = O.moe_layer_token(xc[b], hl.router, hl.expert, wl.k, hl.shared)
        hl._experts.clear()
        worst = max(worst, rel_err(yc[b], y_ref))
    print(f"{name} B={B}: sampled {sample}, worst max|dy|/||y||inf = {worst:.3e}")
    assert worst <= _tol(wl)
    L.close()
    del L
    torch.cuda.empty_cache()


def test_batched_bad_ids_skipped():
    """Given ids with a repeat, an id past E and a negative id (tokens 0-2) at B=16: skipped,
    reported, and y equals the oracle with those choices removed, after a clean call."""
    import torch
    wl = SMALL[0]
    B = 16
    L = _layer(wl, max_batch=B)
    hl = HostLayer(wl)
    attempts, X = _batch(wl, hl, B, case=6)
    ys, ids, ws = _oracle(wl, hl, X)
    x = T.device_x(wl, list(range(B)), attempts=attempts, case=6)
    ids_np = np.stack([ids[b] for b in range(B)]).astype(np.int32)
    w_np = np.stack([ws[b] for b in range(B)]).astype(np.float32)
    w_t = torch.from_numpy(w_np).cuda()
    y = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
    L.forward(x, y, ids=torch.from_numpy(ids_np).cuda(), w=w_t)
    assert L.check() == 0
    bad = corrupt(ids_np, wl.E)
    L.forward(x, y, ids=torch.from_numpy(bad).cuda(), w=w_t)
    assert L.check() != 0
    yc = y.cpu().numpy()
    for b in range(B):
        use = _used(bad[b].tolist(), wl.E)
        y_ref = O.moe_layer_given(X[b], bad[b, use], w_np[b, use], hl.expert, hl.shared)
        assert rel_err(yc[b], y_ref) <= TOL_BF16, b
