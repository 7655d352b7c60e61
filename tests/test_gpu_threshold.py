"""GPU parity of the threshold keep rule (moe_channel_select_threshold) and of the score
read-back (moe_layer_scores) against the oracle: kept ids and their count exactly, y within
tolerance, at small ragged shapes (both score modes, tau between two scores with a margin,
tau at or below zero, tau above every score) and at the full shapes."""
import numpy as np
import pytest

from gpu_common import CH_MARGIN_REL, HostLayer, MARGIN, TOL_BF16, cuda_ok, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O
from test_gpu_channel import MODES, SMALL, _layer

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _draw(wl, hl, token, mode, keep, layer=0):
    """First redraw of x with a router margin and a gap of at least the channel margin
    between the keep-th and (keep+1)-th scores; tau is their midpoint."""
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
        if srt[keep - 1] - srt[keep] < 2 * CH_MARGIN_REL * srt[0]:
            continue
        return x, ids[0], w[0], s, dnorm_of, 0.5 * (srt[keep - 1] + srt[keep])
    raise RuntimeError("no margin-satisfying draw")


def _run(L, wl, x_np, tau, mode):
    import torch
    n = wl.k * wl.I
    x = torch.from_numpy(np.asarray(x_np, dtype=np.float32)).cuda().reshape(1, -1)
    y = torch.empty_like(x)
    kept = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    L.channel_select_threshold(x, tau, kept, cnt, y=y, mode=mode)
    scores = torch.empty(n, dtype=torch.float32, device="cuda")
    L.scores(scores)
    assert L.check() == 0
    c = int(cnt.item())
    return kept.cpu().numpy()[:c], c, y.cpu().numpy()[0], scores.cpu().numpy()


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}{w.expert_dtype}")
def test_threshold_small(wl, mode):
    L = _layer(wl)
    hl = HostLayer(wl)
    n = wl.k * wl.I
    for tok, keep in enumerate([1, n // 8, n // 3 + 1, n - 1]):
        x, ids, w, s, dnorm_of, tau = _draw(wl, hl, 20 + tok, mode, keep)
        kept_ref, y_ref = O.channel_select_threshold_token(x, ids, w, hl.expert, dnorm_of, tau,
                                                           hl.shared, mode)
        assert kept_ref.size == keep
        kept, cnt, y, sc = _run(L, wl, x, tau, MODES[mode])
        assert cnt == keep, (tok, cnt, keep)
        assert kept.tolist() == kept_ref.tolist(), tok
        assert rel_err(y, y_ref) <= TOL_BF16, (tok, rel_err(y, y_ref))
        # the read-back scores: slot-major in routing order
        assert np.max(np.abs(sc - s.ravel())) <= 1e-5 * np.max(s), tok
    # extremes: everything, then nothing
    x, ids, w, s, dnorm_of, _ = _draw(wl, hl, 30, mode, 1)
    kept, cnt, y, _ = _run(L, wl, x, 0.0, MODES[mode])
    kept_ref, y_ref = O.channel_select_token(x, ids, w, hl.expert, dnorm_of, n, hl.shared, mode)
    assert cnt == n and kept.tolist() == kept_ref.tolist()
    assert rel_err(y, y_ref) <= TOL_BF16
    kept, cnt, y, _ = _run(L, wl, x, 1e30, MODES[mode])
    _, y_ref = O.channel_select_token(x, ids, w, hl.expert, dnorm_of, 0, hl.shared, mode)
    assert cnt == 0 and rel_err(y, y_ref) <= TOL_BF16


def test_threshold_full_size():
    """The stack's shapes (H=2048, E=256, k=8, I=768, one shared expert), tau between the
    799th and 800th scores of each token."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    L = _layer(wl, 2)
    hl = HostLayer(wl, 2)
    for tok in (0, 5):
        x, ids, w, s, dnorm_of, tau = _draw(wl, hl, tok, "router_weighted", 799, layer=2)
        kept_ref, y_ref = O.channel_select_threshold_token(x, ids, w, hl.expert, dnorm_of, tau,
                                                           hl.shared, "router_weighted")
        kept, cnt, y, sc = _run(L, wl, x, tau, 1)
        assert cnt == 799 and kept.tolist() == kept_ref.tolist(), tok
        err = rel_err(y, y_ref)
        print(f"threshold token {tok}: max|dy|/||y||inf = {err:.3e}")
        assert err <= TOL_BF16
        assert np.max(np.abs(sc - s.ravel())) <= 1e-5 * np.max(s)
    L.close()
    del L
    torch.cuda.empty_cache()
