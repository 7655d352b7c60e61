"""GPU parity of batch-wide channel selection (moe_channel_select_batch) against the oracle:
kept ids and their count exactly (entries past the count -1), y of every token within
tolerance, at small ragged shapes for B = 1, 4, 8 and 16 (keep at several fractions with a gap
between the keep-th and (keep+1)-th batch scores, keep 0, keep past the candidates), with the
routing given and routed inside the call, and at the full shapes for B = 4, 8 and 16."""
import numpy as np
import pytest

from gpu_common import CH_MARGIN_REL, MARGIN, TOL_BF16, HostLayer, cuda_ok, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O
from test_gpu_channel import SMALL

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _layer(wl, layer=0, max_batch=16):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=max_batch)
    return M.Layer(desc, T.device_layer(wl, layer))


def _batch(wl, hl, B, first, layer=0):
    """B tokens, each the first redraw with a top-k router margin, routed by the oracle."""
    X, ids, w = [], [], []
    for b in range(B):
        for a in range(64):
            x = T.x(wl, first + b, layer, a)
            logits = O.router_logits(x, hl.router)[0]
            if O.topk_margin(logits, wl.k) >= MARGIN:
                break
        else:
            raise RuntimeError("no margin-satisfying draw")
        i, ww = O.route(logits[None], wl.k)
        X.append(x)
        ids.append(i[0])
        w.append(ww[0])
    return np.stack(X), np.stack(ids), np.stack(w)


def _dnorm(hl):
    dn = {}

    def dnorm_of(e):
        if e not in dn:
            dn[e] = O.down_norms(hl.expert(e)[2])
        return dn[e]

    return dnorm_of


def _keeps(sv, wanted):
    """For each wanted keep, the nearest keep in [1, m) whose keep-th and (keep+1)-th batch
    scores differ by the channel margin (the two sides order candidates alike there)."""
    srt = np.sort(sv)[::-1]
    m = srt.size
    gap = 2 * CH_MARGIN_REL * srt[0]
    out = []
    for want in wanted:
        want = min(max(want, 1), m - 1)
        for d in range(m):
            hit = [c for c in (want - d, want + d) if 1 <= c < m and srt[c - 1] - srt[c] >= gap]
            if hit:
                out.append(hit[0])
                break
    return out


def _run(L, wl, X, keep, ids=None, w=None):
    import torch
    B = X.shape[0]
    x = torch.from_numpy(np.asarray(X, dtype=np.float32)).cuda().contiguous()
    y = torch.empty_like(x)
    kept = torch.full((max(keep, 1),), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    ti = None if ids is None else torch.from_numpy(ids.astype(np.int32)).cuda()
    tw = None if w is None else torch.from_numpy(np.asarray(w, np.float32)).cuda()
    L.channel_select_batch(x, keep, kept, y, kept_count=cnt, ids=ti, w=tw)
    assert L.check() == 0
    return kept.cpu().numpy()[:keep], int(cnt.item()), y.cpu().numpy()


def _check(L, wl, hl, X, ids, w, keep, given=True):
    dnorm_of = _dnorm(hl)
    kept_ref, Y_ref = O.batch_channel_select(X, ids, w, hl.expert, dnorm_of, keep, hl.shared)
    kept, cnt, Y = _run(L, wl, X, keep, ids if given else None, w if given else None)
    assert cnt == kept_ref.size, (keep, cnt, kept_ref.size)
    assert kept[:cnt].tolist() == kept_ref.tolist(), keep
    assert np.all(kept[cnt:] == -1), keep
    for b in range(X.shape[0]):
        assert rel_err(Y[b], Y_ref[b]) <= TOL_BF16, (keep, b, rel_err(Y[b], Y_ref[b]))


@pytest.mark.parametrize("B", [1, 4, 8, 16])
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}{w.expert_dtype}")
def test_batch_select_small(wl, B):
    L = _layer(wl)
    hl = HostLayer(wl)
    X, ids, w = _batch(wl, hl, B, 40)
    cid, sv, _ = O.batch_channel_scores(X, ids, w, hl.expert, _dnorm(hl))
    m = cid.size
    for keep in _keeps(sv, [1, m // 8, m // 3 + 1, m - 1]):
        _check(L, wl, hl, X, ids, w, keep)
    # every candidate, keep past the touched candidates, nothing
    _check(L, wl, hl, X, ids, w, m)
    maxcand = min(wl.E, B * wl.k) * wl.I
    _check(L, wl, hl, X, ids, w, maxcand)
    _check(L, wl, hl, X, ids, w, 0)
    L.close()


@pytest.mark.parametrize("wl", SMALL[:2], ids=lambda w: f"H{w.H}E{w.E}k{w.k}I{w.I}")
def test_batch_select_routed_inside(wl):
    """ids = NULL: the layer routes the batch itself (tokens drawn with a router margin)."""
    L = _layer(wl)
    hl = HostLayer(wl)
    X, ids, w = _batch(wl, hl, 5, 60)
    cid, sv, _ = O.batch_channel_scores(X, ids, w, hl.expert, _dnorm(hl))
    for keep in _keeps(sv, [cid.size // 4]):
        _check(L, wl, hl, X, ids, w, keep, given=False)
    L.close()


def test_batch_select_rejects():
    import routed_expert_ffn_route_amd as M
    import torch
    wl = SMALL[0]
    L = _layer(wl, max_batch=4)
    x = torch.zeros((5, wl.H), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    kept = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MoeError):  # B above max_batch
        L.channel_select_batch(x, 4, kept, y)
    with pytest.raises(M.MoeError):  # keep above min(E, B*k)*I
        L.channel_select_batch(x[:1], wl.k * wl.I + 1, kept, y[:1])
    L.close()


@pytest.mark.parametrize("B", [4, 8, 16])
def test_batch_select_full_size(B):
    """The stack's shapes (H=2048, E=256, k=8, I=768, one shared expert) at B = 4, 8, 16 (the
    selection's register layouts for up to 24, 48 and 96 thousand candidates), keep = B * 799
    (the per-token budget times the batch) moved to the nearest score gap."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    L = _layer(wl, 2, max_batch=B)
    hl = HostLayer(wl, 2)
    X, ids, w = _batch(wl, hl, B, 100 + B, layer=2)
    cid, sv, _ = O.batch_channel_scores(X, ids, w, hl.expert, _dnorm(hl))
    (keep,) = _keeps(sv, [B * 799])
    dnorm_of = _dnorm(hl)
    kept_ref, Y_ref = O.batch_channel_select(X, ids, w, hl.expert, dnorm_of, keep, hl.shared)
    kept, cnt, Y = _run(L, wl, X, keep, ids, w)
    assert cnt == keep and kept.tolist() == kept_ref.tolist()
    err = max(rel_err(Y[b], Y_ref[b]) for b in range(B))
    print(f"batch select B={B} keep={keep} of {cid.size}: max rel err {err:.3e}")
    assert err <= TOL_BF16
    L.close()
    del L
    torch.cuda.empty_cache()


def test_batch_select_ties_at_threshold():
    """Equal batch scores straddling the keep-th place: four channels of one touched expert are
    given the same gate and down rows (so both sides compute the same score for each of
    them, bit for bit on the GPU), and keep is set so that only the first two of them are
    kept; both sides keep the lower candidates (e*I + j) of a tie."""
    import torch
    import routed_expert_ffn_route_amd as M
    wl = SMALL[-1]
    hl = HostLayer(wl)
    X, ids, w = _batch(wl, hl, 4, 140)
    touched = sorted(set(int(e) for e in ids.ravel()))
    e0 = touched[len(touched) // 2]
    dev = T.device_layer(wl, 0)
    base = {e: hl.expert(e) for e in touched}
    for j0 in range(0, wl.I - 4, 5):
        mod = {}
        for e in touched:
            # storage form: (dtype tag, rows [I][H])
            g, v, d = ((a[0], np.array(a[1], copy=True)) for a in base[e])
            if e == e0:
                for arr in (g[1], d[1]):
                    arr[j0 + 1:j0 + 4] = arr[j0]
            mod[e] = (g, v, d)
        get = lambda e: mod[e] if e in mod else hl.expert(e)
        dn = {}

        def dnorm_of(e):
            if e not in dn:
                dn[e] = O.down_norms(get(e)[2])
            return dn[e]

        cid, sv, _ = O.batch_channel_scores(X, ids, w, get, dnorm_of)
        tie = sv[np.searchsorted(cid, e0 * wl.I + j0)]
        above = int(np.sum(sv > tie))
        others = sv[sv != tie]
        # the tied value is apart from every other score by the channel margin
        if np.all(np.abs(others - tie) >= 2 * CH_MARGIN_REL * sv.max()):
            break
    else:
        pytest.skip("no isolated score to tie")
    r0 = e0 * wl.I + j0
    for key in ("gate", "down_t"):
        dev[key][r0 + 1:r0 + 4] = dev[key][r0]
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=16)
    L = M.Layer(desc, dev)
    torch.cuda.synchronize()
    keep = above + 2  # two of the four tied channels
    kept_ref, Y_ref = O.batch_channel_select(X, ids, w, get, dnorm_of, keep, hl.shared)
    assert e0 * wl.I + j0 + 1 in kept_ref.tolist() and e0 * wl.I + j0 + 2 not in kept_ref
    kept, cnt, Y = _run(L, wl, X, keep, ids, w)
    assert cnt == keep and kept.tolist() == kept_ref.tolist()
    for b in range(X.shape[0]):
        assert rel_err(Y[b], Y_ref[b]) <= TOL_BF16, (b, rel_err(Y[b], Y_ref[b]))
    L.close()
