"""Property tests (hypothesis, CPU only): the plain C++17 oracle against the numpy oracle over
random tiny shapes and storage types, and invariants of the definitions that hold at any
shape (keep-all equals dense, expert relabelling only relabels ids)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import cpp_oracle as C
from oracle import moe_oracle as O

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


def _stored(rng, rows, cols, dtype):
    a = rng.normal(0, 0.5, (rows, cols))
    if dtype == "f64":
        return a
    if dtype == "f32":
        return a.astype(np.float32)
    return ("bf16", (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))


@st.composite
def layers(draw):
    E = draw(st.integers(1, 8))
    return dict(H=draw(st.integers(1, 12)), E=E, k=draw(st.integers(1, E)),
                I=draw(st.integers(1, 6)), ns=draw(st.integers(0, 2)),
                Is=draw(st.integers(1, 5)), dtype=draw(st.sampled_from(["f64", "f32", "bf16"])),
                seed=draw(st.integers(0, 2**31 - 1)), B=draw(st.integers(1, 4)))


def _build(p):
    rng = np.random.default_rng(p["seed"])
    H, E, I = p["H"], p["E"], p["I"]
    x = rng.normal(size=(p["B"], H))
    Wr = _stored(rng, E, H, p["dtype"])
    ex = [tuple(_stored(rng, I, H, p["dtype"]) for _ in range(3)) for _ in range(E)]
    sh = [tuple(_stored(rng, p["Is"], H, p["dtype"]) for _ in range(3))
          for _ in range(p["ns"])]
    return x, Wr, ex, sh


def _close(a, b, rel=1e-12):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b), initial=0.0) <= rel * max(1.0, np.max(np.abs(b), initial=0.0))


@SETTINGS
@given(layers())
def test_cpp_matches_numpy_layer_and_routing(p):
    x, Wr, ex, sh = _build(p)
    lc = C.router_logits(x, Wr)
    ln = O.router_logits(x, Wr)
    assert _close(lc, ln)
    ids_c, w_c = C.route(ln, p["k"])
    ids_n, w_n = O.route(ln, p["k"])
    assert np.array_equal(ids_c, ids_n)
    assert _close(w_c, w_n, 1e-14)
    for b in range(p["B"]):
        yc, ic, _ = C.moe_layer_token(x[b], Wr, lambda e: ex[e], p["k"], sh, logits=ln[b])
        yn, inn, _ = O.moe_layer_token(x[b], Wr, lambda e: ex[e], p["k"], sh, logits=ln[b])
        assert np.array_equal(ic, inn)
        assert _close(yc, yn)
    n_c = C.union_experts(ids_n, p["E"])
    n_n = O.union_experts(ids_n, p["E"])
    assert n_c[0] == n_n[0] and all(np.array_equal(u, v) for u, v in zip(n_c[1:], n_n[1:]))


@SETTINGS
@given(layers(), st.data())
def test_cpp_matches_numpy_channel_select(p, data):
    x, Wr, ex, sh = _build(p)
    ids, w = O.route(O.router_logits(x[0], Wr), p["k"])
    keep = data.draw(st.integers(0, p["k"] * p["I"]))
    mode = data.draw(st.sampled_from(["gate_dnorm", "router_weighted"]))
    kc, yc = C.channel_select_token(x[0], ids[0], w[0], lambda e: ex[e],
                                    lambda e: C.down_norms(ex[e][2]), keep, sh, mode)
    kn, yn = O.channel_select_token(x[0], ids[0], w[0], lambda e: ex[e],
                                    lambda e: O.down_norms(ex[e][2]), keep, sh, mode)
    assert np.array_equal(kc, kn)
    assert _close(yc, yn)


@SETTINGS
@given(layers())
def test_keep_all_is_dense_and_relabelling_relabels(p):
    """Invariants of the definitions, on the C++ oracle: keeping all k*I channels gives the
    dense layer; renaming the experts by a permutation only renames the chosen ids."""
    x, Wr, ex, sh = _build(p)
    y, ids, w = C.moe_layer_token(x[0], Wr, lambda e: ex[e], p["k"], sh)
    kept, ys = C.channel_select_token(x[0], ids, w, lambda e: ex[e],
                                      lambda e: C.down_norms(ex[e][2]), p["k"] * p["I"], sh)
    assert _close(ys, y, 1e-11)
    assert kept.tolist() == sorted(int(e) * p["I"] + j for e in ids for j in range(p["I"]))
    perm = np.random.default_rng(p["seed"] + 1).permutation(p["E"])
    Wr_p = Wr[perm] if not isinstance(Wr, tuple) else ("bf16", Wr[1][perm])
    y2, ids2, _ = C.moe_layer_token(x[0], Wr_p, lambda e: ex[perm[e]], p["k"], sh)
    assert perm[ids2].tolist() == ids.tolist()
    assert _close(y2, y, 1e-11)


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_cpp_thread_split_does_not_change_results(threads):
    rng = np.random.default_rng(5)
    H, E, k, I = 40, 9, 3, 17
    x = rng.normal(size=H)
    Wr = rng.normal(size=(E, H))
    ex = [tuple(rng.normal(size=(I, H)) for _ in range(3)) for _ in range(E)]
    sh = [tuple(rng.normal(size=(5, H)) for _ in range(3))]
    C.set_threads(1)
    y1, _, _ = C.moe_layer_token(x, Wr, lambda e: ex[e], k, sh)
    C.set_threads(threads)
    try:
        yt, _, _ = C.moe_layer_token(x, Wr, lambda e: ex[e], k, sh)
    finally:
        C.set_threads(1)
    assert np.array_equal(y1, yt)
