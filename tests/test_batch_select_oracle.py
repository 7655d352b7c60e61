"""Pins of the batch-wide channel selection's oracle (CPU only), each tying it to a pinned
oracle or to its definition: one token is the per-token top-K rule in the router-weighted
mode; keeping every candidate is the dense layer for every token; keeping none leaves the
shared experts; a batch of identical tokens keeps that token's top-K set; the kept set is the
top-K of summed scores by brute force over subsets.

Source: the jaehun.me review of arXiv:2610.37386, "Limits" (batch-wide selection is the
authors' future work) and "Background: channels and keep rules"."""
import itertools

import numpy as np

from oracle import moe_oracle as O


def _layer(rng, E=5, I=4, H=6):
    experts = [tuple(rng.normal(0, 0.4, size=(I, H)) for _ in range(3)) for _ in range(E)]
    shared = [tuple(rng.normal(0, 0.4, size=(3, H)) for _ in range(3))]
    dn = {e: O.down_norms(experts[e][2]) for e in range(E)}
    return experts, shared, dn


def _route(rng, B, E, k, H):
    X = rng.normal(size=(B, H))
    logits = rng.normal(size=(B, E))
    ids, w = O.route(logits, k)
    return X, ids, w


def test_one_token_is_the_per_token_rule():
    rng = np.random.default_rng(31)
    experts, shared, dn = _layer(rng)
    X, ids, w = _route(rng, 1, 5, 2, 6)
    for keep in (0, 1, 3, 8):
        kb, Yb = O.batch_channel_select(X, ids, w, lambda e: experts[e], dn.__getitem__, keep,
                                        shared)
        kt, yt = O.channel_select_token(X[0], ids[0], w[0], lambda e: experts[e],
                                        dn.__getitem__, keep, shared, "router_weighted")
        assert kb.tolist() == kt.tolist()
        assert np.allclose(Yb[0], yt, rtol=0, atol=1e-12)


def test_keep_all_is_dense_and_keep_none_is_shared():
    rng = np.random.default_rng(32)
    experts, shared, dn = _layer(rng)
    X, ids, w = _route(rng, 4, 5, 2, 6)
    n_t = len(set(ids.ravel().tolist()))
    kb, Yb = O.batch_channel_select(X, ids, w, lambda e: experts[e], dn.__getitem__, n_t * 4,
                                    shared)
    assert kb.size == n_t * 4
    for b in range(4):
        dense = O.moe_layer_given(X[b], ids[b], w[b], lambda e: experts[e], shared)
        assert np.allclose(Yb[b], dense, rtol=0, atol=1e-12)
    kb, Yb = O.batch_channel_select(X, ids, w, lambda e: experts[e], dn.__getitem__, 0, shared)
    assert kb.size == 0
    for b in range(4):
        sh = sum(O.expert_output(X[b], *t) for t in shared)
        assert np.allclose(Yb[b], sh, rtol=0, atol=1e-12)


def test_identical_tokens_keep_the_tokens_top_k():
    rng = np.random.default_rng(33)
    experts, shared, dn = _layer(rng)
    X, ids, w = _route(rng, 1, 5, 3, 6)
    Xb, idsb, wb = np.repeat(X, 3, 0), np.repeat(ids, 3, 0), np.repeat(w, 3, 0)
    for keep in (1, 5, 9):
        kb, Yb = O.batch_channel_select(Xb, idsb, wb, lambda e: experts[e], dn.__getitem__,
                                        keep, shared)
        kt, yt = O.channel_select_token(X[0], ids[0], w[0], lambda e: experts[e],
                                        dn.__getitem__, keep, shared, "router_weighted")
        assert kb.tolist() == kt.tolist()
        for b in range(3):
            assert np.allclose(Yb[b], yt, rtol=0, atol=1e-12)


def test_kept_set_is_the_best_summed_scores_by_brute_force():
    rng = np.random.default_rng(34)
    experts, shared, dn = _layer(rng, E=4, I=2, H=5)
    X, ids, w = _route(rng, 3, 4, 2, 5)
    touched = sorted(set(ids.ravel().tolist()))
    total = {}
    for e in touched:
        for j in range(2):
            t = 0.0
            for b in range(3):
                hit = np.nonzero(ids[b] == e)[0]
                if hit.size:
                    g = experts[e][0][j] @ X[b]
                    t += w[b, hit[0]] * dn[e][j] * abs(g / (1 + np.exp(-g)))
            total[e * 2 + j] = t
    cands = sorted(total)
    for keep in range(len(cands) + 1):
        best = max(itertools.combinations(cands, keep), key=lambda sub: sum(total[c] for c in sub))
        kb, _ = O.batch_channel_select(X, ids, w, lambda e: experts[e], dn.__getitem__, keep,
                                       shared)
        assert kb.tolist() == sorted(best)
