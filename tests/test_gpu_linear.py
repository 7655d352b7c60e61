"""GPU parity of routing from given logits, the touched-expert union, and the linear-expert
(one matrix per expert) batched layer on MFMA, against the oracle."""
import numpy as np
import pytest

from gpu_common import TOL_BF16, corrupt, cuda_ok, rel_err, used_choices as _used
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _layer(wl, max_batch):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, kind=M.LINEAR, router_dtype=None,
                       expert_dtype="bf16", max_batch=max_batch)
    return M.Layer(desc, T.device_layer(wl, 0))


def _route_given_logits(L, wl, tokens, case):
    import torch
    logits = T.device_logits(wl, tokens, case=case)
    B = len(tokens)
    ids = torch.empty((B, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, wl.k), dtype=torch.float32, device="cuda")
    L.route(logits_in=logits, ids=ids, w=w)
    return logits, ids, w


@pytest.mark.parametrize("E,k,B", [(16, 3, 1), (64, 3, 16), (64, 3, 256), (8, 2, 4096),
                                   (896, 16, 16), (5, 5, 7), (3000, 8, 33)])
def test_union_matches_oracle(E, k, B):
    import torch
    import routed_expert_ffn_route_amd as M
    rng = np.random.default_rng(E * 1000 + B)
    ids_np = np.stack([rng.choice(E, k, replace=False) for _ in range(B)]).astype(np.int32)
    ids = torch.from_numpy(ids_np).cuda()
    n_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    touched = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    slots = torch.zeros(B * k, dtype=torch.int32, device="cuda")
    M.union_experts(ids, E, n_t, touched, offsets, slots)
    n_ref, t_ref, o_ref, s_ref = O.union_experts(ids_np, E)
    assert int(n_t.item()) == n_ref
    assert touched.cpu().numpy()[:n_ref].tolist() == t_ref.tolist()
    assert offsets.cpu().numpy().tolist() == o_ref.tolist()
    assert slots.cpu().numpy().tolist() == s_ref.tolist()


SMALL = [
    T.reduced(WORKLOADS["linear_e64_k3"], wid=131, H=1024, E=7, k=2, I=96),
    T.reduced(WORKLOADS["linear_e64_k3"], wid=132, H=2048, E=16, k=3, I=256),
]


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 16, 31, 40, 300, 600])
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}")
def test_linear_small(wl, B):
    import torch
    L = _layer(wl, max_batch=600)
    tokens = list(range(B))
    logits, ids, w = _route_given_logits(L, wl, tokens, case=1)
    lg = logits.cpu().numpy()
    ids_ref, w_ref = O.route(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) < 1e-6
    x = T.device_x(wl, tokens, case=1)
    y = torch.empty((B, wl.I), dtype=torch.float32, device="cuda")
    L.forward(x, y, ids=ids, w=w)
    assert L.check() == 0
    mats = {}

    def get(e):
        if e not in mats:
            mats[e] = T.linear(wl, e)
        return mats[e]

    Y = O.linear_moe(x.cpu().numpy(), ids_ref, w_ref, get)
    err = rel_err(y.cpu().numpy(), Y)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("B", [1, 4, 16, 64, 256, 2048])
def test_linear_full_size_sampled(B):
    """E=64, k=3, 8192x8192 bf16 experts; every batch size of the sweep, sampled tokens."""
    import torch
    wl = WORKLOADS["linear_e64_k3"]
    L = _layer(wl, max_batch=2048)
    tokens = list(range(B))
    logits, ids, w = _route_given_logits(L, wl, tokens, case=2)
    ids_ref, w_ref = O.route(logits.cpu().numpy(), wl.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    x = T.device_x(wl, tokens, case=2)
    y = torch.empty((B, wl.I), dtype=torch.float32, device="cuda")
    L.forward(x, y, ids=ids, w=w)
    assert L.check() == 0
    sample = sorted(set([0, B - 1, B // 2, B // 3]))
    mats = {}

    def get(e):
        if e not in mats:
            mats[e] = T.linear(wl, e)
        return mats[e]

    xs = x.cpu().numpy()
    ys = y.cpu().numpy()
    worst = 0.0
    for b in sample:
        yref = O.linear_moe(xs[b:b + 1], ids_ref[b:b + 1], w_ref[b:b + 1], get)[0]
        worst = max(worst, rel_err(ys[b], yref))
    print(f"B={B}: sampled tokens {sample}, worst max|dy|/||y||inf = {worst:.3e}")
    assert worst <= TOL_BF16
    L.close()
    del L
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_linear_small_batch_flags_bad_ids():
    """At B <= 4 the VALU kernel reads the ids itself: an id repeated within a token or
    outside [0, E) is skipped and reported through the layer's error bits; a clean call
    afterwards reports nothing."""
    import torch
    wl = SMALL[1]
    L = _layer(wl, max_batch=4)
    x = T.device_x(wl, [0, 1], case=1)
    y = torch.empty((2, wl.I), dtype=torch.float32, device="cuda")
    w = torch.full((2, wl.k), 1.0 / wl.k, dtype=torch.float32, device="cuda")
    for bad in ([[1, 1, 2], [3, 4, 5]], [[1, 2, wl.E], [3, 4, 5]]):
        ids = torch.tensor(bad, dtype=torch.int32, device="cuda")
        L.forward(x, y, ids=ids, w=w)
        assert L.check() != 0
    ids = torch.tensor([[1, 2, 3], [3, 4, 5]], dtype=torch.int32, device="cuda")
    L.forward(x, y, ids=ids, w=w)
    assert L.check() == 0


@pytest.mark.parametrize("B", [3, 16, 40])
def test_linear_bad_ids_skipped_every_path(B):
    """Bad given ids at B=3 (VALU row-owner kernel), B=16 (VALU passes) and B=40 (MFMA
    tiles): the bad choices are skipped, the error word is set, and y equals the oracle with
    those choices removed -- also after a clean call has left other partial rows behind."""
    import torch
    wl = SMALL[1]
    L = _layer(wl, max_batch=64)
    tokens = list(range(B))
    logits, ids, w = _route_given_logits(L, wl, tokens, case=5)
    x = T.device_x(wl, tokens, case=5)
    y = torch.empty((B, wl.I), dtype=torch.float32, device="cuda")
    L.forward(x, y, ids=ids, w=w)  # a clean call first: partial rows of every choice written
    assert L.check() == 0
    bad = corrupt(ids.cpu().numpy(), wl.E)
    L.forward(x, y, ids=torch.from_numpy(bad).cuda(), w=w)
    assert L.check() != 0
    mats = {}

    def get(e):
        if e not in mats:
            mats[e] = T.linear(wl, e)
        return mats[e]

    xs, ys, wn = x.cpu().numpy(), y.cpu().numpy(), w.cpu().numpy()
    for b in range(B):
        use = _used(bad[b].tolist(), wl.E)
        yref = O.linear_moe(xs[b:b + 1], bad[b:b + 1, use], wn[b:b + 1, use], get)[0]
        assert rel_err(ys[b], yref) <= TOL_BF16, b
