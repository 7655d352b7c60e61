"""GPU parity of the batch-1 layer with MXFP4 routed experts (bf16 router and shared
experts) against the oracle, which dequantises the same codes and scales exactly."""
import numpy as np
import pytest

from gpu_common import HostLayer, TOL_MXFP4, cuda_ok, pick_attempt, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _layer(wl, layer=0, max_batch=1):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=max_batch)
    return M.Layer(desc, T.device_layer(wl, layer))


W_TOL = 1e-6  # router weights of the launch vs the oracle's fp64 softmax


def _routing(L, k, B=1):
    import torch
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, k), dtype=torch.float32, device="cuda")
    L.routing(ids, w, B=B)
    return ids.cpu().numpy(), w.cpu().numpy()


def _run(L, x_np):
    import torch
    x = torch.from_numpy(x_np).cuda().reshape(1, -1)
    y = torch.empty_like(x)
    L.forward(x, y)
    assert L.check() == 0
    return y.cpu().numpy()[0]


SMALL = [
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=141, H=1024, E=40, k=4, I=96, n_shared=2,
              I_shared=64, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=142, H=7168, E=64, k=16, I=40, n_shared=1,
              I_shared=24, layers=1),
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=143, H=2048, E=17, k=3, I=200, n_shared=0,
              I_shared=0, layers=1),
    # long expert rows (I = 32800) and a share of more than 512 routed channels per
    # workgroup
    T.reduced(WORKLOADS["mxfp4_e896_k16"], wid=144, H=256, E=4, k=4, I=32800, n_shared=1,
              I_shared=64, layers=1),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}s{w.n_shared}")
def test_mxfp4_b1_small(wl):
    L = _layer(wl)
    hl = HostLayer(wl)
    for tok in range(3):
        a, x = pick_attempt(wl, tok, host_router=hl.router)
        y_ref, _, _ = O.moe_layer_token(x, hl.router, hl.expert, wl.k, hl.shared)
        y = _run(L, x)
        err = rel_err(y, y_ref)
        assert err <= TOL_MXFP4, (tok, err)


def test_mxfp4_b1_full_size_sampled():
    """H=7168, E=896, k=16, I=2048, two shared experts: one layer, two tokens."""
    import torch
    wl = WORKLOADS["mxfp4_e896_k16"]
    L = _layer(wl, 0)
    hl = HostLayer(wl, 0)
    for tok in (0, 5):
        a, x = pick_attempt(wl, tok, 0, host_router=hl.router)
        y_ref, ids_ref, w_ref = O.moe_layer_token(x, hl.router, hl.expert, wl.k, hl.shared)
        hl._experts.clear()
        y = _run(L, x)
        rid, rw = _routing(L, wl.k)
        assert rid[0].tolist() == ids_ref.tolist()
        assert np.max(np.abs(rw[0] - w_ref)) <= W_TOL
        err = rel_err(y, y_ref)
        print(f"mxfp4 token {tok}: max|dy|/||y||inf = {err:.3e}")
        assert err <= TOL_MXFP4
    L.close()
    del L
    torch.cuda.empty_cache()


def test_mxfp4_routing_full_size_tokens():
    """E=896, k=16 routing at the full shapes for 10 margin-checked tokens over two layers:
    the top-k the single launch chose (moe_layer_routing after moe_ffn_forward) and that of
    moe_route, both against the oracle's ids in routing order and its weights."""
    import torch
    wl = WORKLOADS["mxfp4_e896_k16"]
    for layer in (0, 5):
        L = _layer(wl, layer)
        Wr = T.router(wl, layer)
        for tok in range(5):
            a, x = pick_attempt(wl, tok, layer, host_router=Wr)
            ids_ref, w_ref = O.route(O.router_logits(x, Wr), wl.k)
            xd = torch.from_numpy(x).cuda().reshape(1, -1)
            ids = torch.empty((1, wl.k), dtype=torch.int32, device="cuda")
            w = torch.empty((1, wl.k), dtype=torch.float32, device="cuda")
            L.route(x=xd, ids=ids, w=w)
            assert ids.cpu().numpy()[0].tolist() == ids_ref[0].tolist(), (layer, tok)
            assert np.max(np.abs(w.cpu().numpy()[0] - w_ref[0])) <= W_TOL
            _run(L, x)
            rid, rw = _routing(L, wl.k)
            assert rid[0].tolist() == ids_ref[0].tolist(), (layer, tok)
            assert np.max(np.abs(rw[0] - w_ref[0])) <= W_TOL
        L.close()
        del L
        torch.cuda.empty_cache()
