"""Pins of the threshold keep rule's oracle (CPU only), each tying it to the top-K rule's
oracle (pinned in test_oracle_pins.py) or to its definition: tau at or below zero keeps every
candidate (the dense layer), a tau above every score keeps none (the shared experts only), a
tau equal to a token's K-th largest score keeps exactly that token's top-K set, the kept set
is {score >= tau} by a plain loop, and the calibrated tau keeps the calibrated fraction of the
pooled calibration candidates.

Source: the jaehun.me review of arXiv:2610.37386, "Background: channels and keep rules" (the
threshold and top-k rows of its table) and the calibration discussion that follows."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _layer(rng, E=5, I=6, H=7, n_shared=1, I_s=3):
    experts = [tuple(rng.normal(0, 0.4, size=(I, H)) for _ in range(3)) for _ in range(E)]
    shared = [tuple(rng.normal(0, 0.4, size=(I_s, H)) for _ in range(3))
              for _ in range(n_shared)]
    dn = {e: O.down_norms(experts[e][2]) for e in range(E)}
    return experts, shared, dn


@pytest.mark.parametrize("mode", ["gate_dnorm", "router_weighted"])
def test_tau_extremes_and_topk_equivalence(mode):
    rng = np.random.default_rng(11)
    experts, shared, dn = _layer(rng)
    get, dnorm_of = (lambda e: experts[e]), dn.__getitem__
    ids, w = np.array([3, 0, 4]), np.array([0.5, 0.3, 0.2])
    x = rng.normal(size=7)
    n = len(ids) * 6
    dense_kept, dense_y = O.channel_select_token(x, ids, w, get, dnorm_of, n, shared, mode)
    kept, y = O.channel_select_threshold_token(x, ids, w, get, dnorm_of, 0.0, shared, mode)
    assert kept.tolist() == dense_kept.tolist() and np.allclose(y, dense_y, rtol=0, atol=1e-12)
    kept, y = O.channel_select_threshold_token(x, ids, w, get, dnorm_of, np.inf, shared, mode)
    assert kept.size == 0
    sh = sum(O.expert_output(x, *t) for t in shared)
    assert np.allclose(y, sh, rtol=0, atol=1e-12)
    s, _ = O.channel_scores(x, ids, w, get, dnorm_of, mode)
    srt = np.sort(s.ravel())[::-1]
    assert np.all(np.diff(srt) < 0)  # distinct
    for K in (1, 4, n - 1):
        tk, ty = O.channel_select_token(x, ids, w, get, dnorm_of, K, shared, mode)
        kept, y = O.channel_select_threshold_token(x, ids, w, get, dnorm_of, srt[K - 1],
                                                   shared, mode)
        assert kept.tolist() == tk.tolist()
        assert np.allclose(y, ty, rtol=0, atol=1e-12)


def test_kept_set_is_the_scores_at_or_above_tau():
    rng = np.random.default_rng(12)
    experts, shared, dn = _layer(rng, E=4, I=5)
    ids, w = np.array([2, 1]), np.array([0.6, 0.4])
    x = rng.normal(size=7)
    s, _ = O.channel_scores(x, ids, w, lambda e: experts[e], dn.__getitem__)
    tau = float(np.median(s))
    kept, _ = O.channel_select_threshold_token(x, ids, w, lambda e: experts[e], dn.__getitem__,
                                               tau, shared)
    want = []
    for i, e in enumerate(ids):
        for j in range(5):
            if s[i, j] >= tau:
                want.append(int(e) * 5 + j)
    assert kept.tolist() == sorted(want)


def test_calibrated_tau_keeps_the_calibrated_fraction():
    rng = np.random.default_rng(13)
    sets = [np.abs(rng.normal(size=(4, 25))) for _ in range(8)]  # 8 tokens x 100 candidates
    for frac in (0.13, 0.18, 0.5):
        tau = O.calibrate_tau(sets, frac)
        kept = sum(int(np.sum(t >= tau)) for t in sets)
        assert kept == int(np.floor(frac * 800 + 0.5))
        # per token the count varies, the pooled mean meets the budget
        per = [int(np.sum(t >= tau)) for t in sets]
        assert abs(np.mean(per) / 100 - frac) <= 0.5 / 800 * 8 + 1e-12
    assert O.calibrate_tau(sets, 0.0) == np.inf
