"""GPU parity of the channel-sparse batch-1 layer (fixed-count top-K keep rule) vs the oracle."""
import numpy as np
import pytest

from gpu_common import CH_MARGIN_REL, HostLayer, MARGIN, TOL_BF16, cuda_ok, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

MODES = {"gate_dnorm": 0, "router_weighted": 1}


def _layer(wl, layer=0):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    return M.Layer(desc, T.device_layer(wl, layer))


def pick_attempt_cs(wl, hl, token, keep, mode, layer=0):
    """First redraw of x with a top-k router margin and a K-th/(K+1)-th score margin."""
    dn = {}

    def dnorm_of(e):
        if e not in dn:
            dn[e] = O.down_norms(hl.expert(e)[2])
        return dn[e]

    for a in range(64):
        x = T.x(wl, token, layer, a)
        logits = O.router_logits(x, hl.router)[0]
        if O.topk_margin(logits, wl.k) < MARGIN:
            continue
        ids, w = O.route(logits[None], wl.k)
        s, _ = O.channel_scores(x, ids[0], w[0], hl.expert, dnorm_of, mode)
        srt = np.sort(s.ravel())[::-1]
        if 0 < keep < srt.size and srt[keep - 1] - srt[keep] < CH_MARGIN_REL * srt[0]:
            continue
        return a, x, dnorm_of
    raise RuntimeError("no margin-satisfying draw")


def _run(L, wl, x_np, keep, mode, ids=None, w=None):
    import torch
    x = torch.from_numpy(x_np).cuda().reshape(1, -1)
    y = torch.empty_like(x)
    kept = torch.full((max(keep, 1),), -1, dtype=torch.int32, device="cuda")
    L.channel_select(x, keep, kept, y=y, ids=ids, w=w, mode=mode)
    assert L.check() == 0
    return kept.cpu().numpy()[:keep], y.cpu().numpy()[0]


SMALL = [
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=111, H=352, E=37, k=5, I=72, n_shared=1,
              I_shared=56, layers=1),
    T.reduced(WORKLOADS["tiny_f32"], wid=112, H=96, E=13, k=3, I=40, n_shared=2, I_shared=24,
              shared_dtype="f32"),
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=113, H=2048, E=64, k=8, I=96, n_shared=1,
              I_shared=128, layers=1),
]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}{w.expert_dtype}")
def test_channel_select_small(wl, mode):
    L = _layer(wl)
    hl = HostLayer(wl)
    n = wl.k * wl.I
    for tok, keep in enumerate([1, 7, n // 8, n // 3 + 1, n - 1]):
        a, x, dnorm_of = pick_attempt_cs(wl, hl, tok, keep, mode)
        ids, w = O.route(O.router_logits(x, hl.router), wl.k)
        kept_ref, y_ref = O.channel_select_token(x, ids[0], w[0], hl.expert, dnorm_of, keep,
                                                 hl.shared, mode)
        kept, y = _run(L, wl, x, keep, MODES[mode])
        assert kept.tolist() == kept_ref.tolist(), (tok, keep)
        assert rel_err(y, y_ref) <= TOL_BF16, (tok, keep, rel_err(y, y_ref))


def test_channel_select_degenerate_keeps():
    """keep = 0 gives the shared experts only; keep = k*I gives the dense layer."""
    import torch
    wl = SMALL[0]
    L = _layer(wl)
    hl = HostLayer(wl)
    a, x, dnorm_of = pick_attempt_cs(wl, hl, 9, 0, "gate_dnorm")
    y_dense, _, _ = O.moe_layer_token(x, hl.router, hl.expert, wl.k, hl.shared)
    y_shared = sum(O.expert_output(x, *s) for s in hl.shared)
    _, y0 = _run(L, wl, x, 0, 0)
    assert rel_err(y0, y_shared) <= TOL_BF16
    n = wl.k * wl.I
    kept, yn = _run(L, wl, x, n, 0)
    ids, _ = O.route(O.router_logits(x, hl.router), wl.k)
    assert kept.tolist() == sorted(int(e) * wl.I + j for e in ids[0] for j in range(wl.I))
    assert rel_err(yn, y_dense) <= TOL_BF16
    # and the dense kernel agrees with keep-everything to fp32 rounding
    xd = torch.from_numpy(x).cuda().reshape(1, -1)
    yd = torch.empty_like(xd)
    L.forward(xd, yd)
    assert rel_err(yn, yd.cpu().numpy()[0]) < 1e-5


def test_channel_select_given_routing_and_repeatable():
    import torch
    wl = SMALL[2]
    L = _layer(wl)
    hl = HostLayer(wl)
    keep = 100
    a, x, dnorm_of = pick_attempt_cs(wl, hl, 3, keep, "gate_dnorm")
    ids, w = O.route(O.router_logits(x, hl.router), wl.k)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w.astype(np.float32)).cuda()
    k1, y1 = _run(L, wl, x, keep, 0, ids=ids_d, w=w_d)
    k2, y2 = _run(L, wl, x, keep, 0, ids=ids_d, w=w_d)
    assert np.array_equal(k1, k2) and np.array_equal(y1, y2)
    kept_ref, y_ref = O.channel_select_token(x, ids[0], w[0], hl.expert, dnorm_of, keep,
                                             hl.shared)
    assert k1.tolist() == kept_ref.tolist()
    assert rel_err(y1, y_ref) <= TOL_BF16


@pytest.mark.parametrize("frac_i", [0, 1])
def test_channel_select_full_size(frac_i):
    """The 40-layer stack's shapes (H=2048, E=256, k=8, I=768, +1 shared) at 13% / 18%."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    keep = wl.keep_counts()[frac_i]
    assert keep == (799, 1106)[frac_i]
    L = _layer(wl, 0)
    hl = HostLayer(wl, 0)
    for tok in (0, 77):
        a, x, dnorm_of = pick_attempt_cs(wl, hl, tok, keep, "gate_dnorm")
        ids, w = O.route(O.router_logits(x, hl.router), wl.k)
        kept_ref, y_ref = O.channel_select_token(x, ids[0], w[0], hl.expert, dnorm_of, keep,
                                                 hl.shared)
        kept, y = _run(L, wl, x, keep, 0)
        assert kept.tolist() == kept_ref.tolist()
        # the top-k the launch chose itself, in routing order
        rid = torch.empty((1, wl.k), dtype=torch.int32, device="cuda")
        rw = torch.empty((1, wl.k), dtype=torch.float32, device="cuda")
        L.routing(rid, rw)
        assert rid.cpu().numpy()[0].tolist() == ids[0].tolist()
        assert np.max(np.abs(rw.cpu().numpy()[0] - w[0])) <= 1e-6
        err = rel_err(y, y_ref)
        print(f"keep {keep} token {tok} attempt {a}: max|dy|/||y||inf = {err:.3e}")
        assert err <= TOL_BF16


def test_channel_select_poisoned_workspace():
    """A workspace whose every 8-byte word carries the first launch's tag (as memory reused
    from an earlier layer can) must not be mistaken for this launch's data: layer creation
    clears every tagged word."""
    import torch
    import routed_expert_ffn_route_amd as M
    wl = SMALL[2]
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    nbytes = (M.workspace_bytes(desc) + 256 + 7) // 8 * 8
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws.view(torch.int64).fill_((1 << 32) | 0x3F800000)  # tag 1, value 1.0
    L = M.Layer(desc, T.device_layer(wl, 0), workspace=ws)
    hl = HostLayer(wl)
    keep = 100
    a, x, dnorm_of = pick_attempt_cs(wl, hl, 5, keep, "gate_dnorm")
    ids, w = O.route(O.router_logits(x, hl.router), wl.k)
    kept_ref, y_ref = O.channel_select_token(x, ids[0], w[0], hl.expert, dnorm_of, keep,
                                             hl.shared)
    kept, y = _run(L, wl, x, keep, 0)
    assert kept.tolist() == kept_ref.tolist()
    assert rel_err(y, y_ref) <= TOL_BF16
