"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test ties one oracle function to something other than itself: a value the pages
print, a closed form, an exact enumeration, brute force on a tiny input written as plain
loops, or an invariant of the definition.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import cpp_oracle as CPP
from oracle import moe_oracle as O

# The pins below that take an `O` argument run against both oracles: the numpy one and the
# plain C++17 one (oracle/cpp/moe_oracle.cpp through oracle/cpp_oracle.py).
both = pytest.mark.parametrize("O", [O, CPP], ids=["numpy", "cpp"])

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- plain-loop references
def loop_expert(x, G, V, Dt):
    """sum_j silu(sum_h G[j,h] x[h]) * (sum_h V[j,h] x[h]) * Dt[j, :], in Python loops."""
    I, H = len(G), len(x)
    y = [0.0] * H
    for j in range(I):
        g = sum(G[j][h] * x[h] for h in range(H))
        u = sum(V[j][h] * x[h] for h in range(H))
        a = g / (1.0 + math.exp(-g)) * u
        for h in range(H):
            y[h] += a * Dt[j][h]
    return y


def rand_expert(rng, I, H, scale=0.5):
    return (rng.normal(0, scale, (I, H)), rng.normal(0, scale, (I, H)),
            rng.normal(0, scale, (I, H)))


# ---------------------------------------------------------------- storage decoding
@both
def test_bf16_widening_known_patterns(O):
    pats = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x3C23], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625, 0.009948730468750]
    assert O.bf16_to_f64(pats).tolist() == want


@both
def test_mxfp4_e2m1_table_and_scale(O):
    # OCP MX v1.0 FP4 E2M1: codes 0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
    codes = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2], dtype=np.uint8)
    vals = O.mxfp4_to_f64(codes, np.array([[127]], dtype=np.uint8))[0]
    mags = [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert vals[:16].tolist() == mags + [-m for m in mags]
    assert O.mxfp4_to_f64(codes, np.array([[130]], dtype=np.uint8))[0][:8].tolist() == \
        [8 * m for m in mags]
    tiny = O.mxfp4_to_f64(codes, np.array([[0]], dtype=np.uint8))[0]
    assert tiny[2] == 2.0 ** -127


@both
def test_mxfp4_generator_roundtrip_bound(O):
    import synth
    codes, scales = synth.mxfp4(0, 123, 0, 4, 256, 0.02)
    w = synth.normal_f32(0, 123, 0, 4 * 256, 0.02).reshape(4, 256).astype(np.float64)
    q = O.mxfp4_to_f64(codes, scales)
    step = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=1)
    # Round to nearest on the grid (spacing <= 2 units) or saturate at 6 from below 8.
    assert np.all(np.abs(q - w) <= 2.0 * step)
    inside = np.abs(w) <= 5.0 * step
    assert np.all(np.abs(q - w)[inside] <= 1.0 * step[inside])
    # values already on the grid come back exactly
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -6, -1.5])
    code = {0: 0, .5: 1, 1: 2, 1.5: 3, 2: 4, 3: 5, 4: 6, 6: 7}
    nib = [code[abs(v)] | (8 if v < 0 else 0) for v in grid] + [0] * 22
    by = np.array([[nib[2 * i] | (nib[2 * i + 1] << 4) for i in range(16)]], dtype=np.uint8)
    assert O.mxfp4_to_f64(by, np.array([[127]], dtype=np.uint8))[0][:10].tolist() == grid.tolist()


# ---------------------------------------------------------------- routing
@both
def test_router_identity_rows_give_x(O):
    rng = np.random.default_rng(1)
    x = rng.normal(size=8)
    assert np.array_equal(O.router_logits(x, np.eye(8))[0], x)


@both
@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (8, 3), (10, 4), (7, 7)])
def test_topk_bruteforce_subsets(E, k, O):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(20):
        l = rng.normal(size=E)
        ids, w = O.route(l[None, :], k)
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(l[i] for i in s))
        assert set(ids[0].tolist()) == set(best)
        assert all(l[ids[0][i]] > l[ids[0][i + 1]] for i in range(k - 1))


@both
def test_topk_exact_ties_go_to_lower_index(O):
    l = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -1.0])
    assert O.route(l[None], 2)[0][0].tolist() == [1, 2]
    assert O.route(l[None], 4)[0][0].tolist() == [1, 2, 4, 3]
    assert O.route(np.zeros((1, 5)), 3)[0][0].tolist() == [0, 1, 2]


@both
def test_softmax_weights_closed_forms(O):
    l = np.array([[2.0, 1.0, 0.0, -3.0]])
    ids, w = O.route(l, 2)
    assert ids[0].tolist() == [0, 1]
    assert w[0] == pytest.approx([math.e / (1 + math.e), 1 / (1 + math.e)], rel=1e-15)
    assert O.route(l, 1)[1][0].tolist() == [1.0]
    assert O.route(np.full((1, 6), 0.3), 4)[1][0] == pytest.approx([0.25] * 4, rel=1e-15)
    # renormalised top-k equals softmax over all E, restricted to the top k and renormalised
    rng = np.random.default_rng(3)
    l = rng.normal(size=(1, 16))
    ids, w = O.route(l, 5)
    full = np.exp(l[0]) / np.exp(l[0]).sum()
    ref = full[ids[0]] / full[ids[0]].sum()
    assert np.max(np.abs(w[0] - ref)) < 1e-12


def test_topk_margin():
    assert O.topk_margin(np.array([5.0, 1.0, 4.5, 0.0]), 2) == pytest.approx(0.5)
    assert O.topk_margin(np.array([5.0, 1.0, 4.5, 0.0]), 1) == pytest.approx(0.5)
    assert O.topk_margin(np.array([5.0, 4.0, 3.0, 2.9]), 3) == pytest.approx(0.1)


# ---------------------------------------------------------------- experts and mixture
@both
def test_swiglu_hand_example(O):
    g = golden("swiglu_hand_example.json")
    x = np.array(g["x"])
    ex = [(np.array(e["G"]), np.array(e["V"]), np.array(e["Dt"])) for e in g["experts"]]
    a = [O.expert_activations(x, G, V)[0] for (G, V, _) in ex]
    assert a == pytest.approx(g["a"], rel=1e-15)
    y = sum(w * O.expert_output(x, *e) for w, e in zip(g["w"], ex))
    assert y.tolist() == pytest.approx(g["y"], rel=1e-15)


@both
def test_expert_output_matches_loops_nonsquare(O):
    rng = np.random.default_rng(4)
    H, I = 7, 5                       # non-square so a transposed operand cannot pass
    x = rng.normal(size=H)
    G, V, Dt = rand_expert(rng, I, H)
    ref = loop_expert(x.tolist(), G.tolist(), V.tolist(), Dt.tolist())
    assert np.max(np.abs(O.expert_output(x, G, V, Dt) - ref)) < 1e-12


@both
def test_k_equals_E_is_dense_softmax_mixture(O):
    rng = np.random.default_rng(5)
    H, I, E = 6, 4, 5
    x = rng.normal(size=H)
    Wr = rng.normal(size=(E, H))
    experts = [rand_expert(rng, I, H) for _ in range(E)]
    sh = rand_expert(rng, I, H)
    y, ids, w = O.moe_layer_token(x, Wr, lambda e: experts[e], E, shared=[sh])
    l = [sum(Wr[e][h] * x[h] for h in range(H)) for e in range(E)]
    z = [math.exp(v - max(l)) for v in l]
    p = [v / sum(z) for v in z]
    ref = np.array(loop_expert(x.tolist(), *[m.tolist() for m in sh]))
    for e in range(E):
        ref += p[e] * np.array(loop_expert(x.tolist(), *[m.tolist() for m in experts[e]]))
    assert sorted(ids.tolist()) == list(range(E))
    assert np.max(np.abs(y - ref)) < 1e-12


@both
def test_top1_of_one_expert_is_textbook_swiglu(O):
    rng = np.random.default_rng(6)
    H, I = 5, 3
    x = rng.normal(size=H)
    ex = rand_expert(rng, I, H)
    y, ids, w = O.moe_layer_token(x, rng.normal(size=(1, H)), lambda e: ex, 1)
    assert ids.tolist() == [0] and w.tolist() == [1.0]
    assert np.max(np.abs(y - loop_expert(x.tolist(), *[m.tolist() for m in ex]))) < 1e-12


@both
def test_zero_gate_leaves_shared_only(O):
    rng = np.random.default_rng(7)
    H, I, E, k = 6, 4, 6, 2
    x = rng.normal(size=H)
    experts = [(np.zeros((I, H)), rng.normal(size=(I, H)), rng.normal(size=(I, H)))
               for _ in range(E)]
    sh = rand_expert(rng, I, H)
    y, _, _ = O.moe_layer_token(x, rng.normal(size=(E, H)), lambda e: experts[e], k,
                                shared=[sh])
    assert np.max(np.abs(y - loop_expert(x.tolist(), *[m.tolist() for m in sh]))) < 1e-12


@both
def test_expert_permutation_only_permutes_ids(O):
    rng = np.random.default_rng(8)
    H, I, E, k = 6, 3, 7, 3
    x = rng.normal(size=H)
    Wr = rng.normal(size=(E, H))
    experts = [rand_expert(rng, I, H) for _ in range(E)]
    perm = rng.permutation(E)          # new expert n is old expert perm[n]
    y0, ids0, w0 = O.moe_layer_token(x, Wr, lambda e: experts[e], k)
    y1, ids1, w1 = O.moe_layer_token(x, Wr[perm], lambda e: experts[perm[e]], k)
    assert perm[ids1].tolist() == ids0.tolist()
    assert np.allclose(w0, w1, rtol=0, atol=1e-15)
    assert np.max(np.abs(y0 - y1)) < 1e-12


# ---------------------------------------------------------------- channel selection
def _sparse_setup(seed, H=5, I=3, E=5, k=2):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=H)
    Wr = rng.normal(size=(E, H))
    experts = [rand_expert(rng, I, H) for _ in range(E)]
    sh = rand_expert(rng, I, H)
    ids, w = O.route(O.router_logits(x, Wr), k)
    return x, experts, sh, ids[0], w[0]


@both
def test_keep_all_channels_equals_dense(O):
    x, experts, sh, ids, w = _sparse_setup(9)
    k, I = len(ids), experts[0][0].shape[0]
    kept, y = O.channel_select_token(x, ids, w, lambda e: experts[e],
                                     lambda e: O.down_norms(experts[e][2]), k * I, shared=[sh])
    dense = sum(we * O.expert_output(x, *experts[e]) for e, we in zip(ids, w))
    dense = dense + O.expert_output(x, *sh)
    assert kept.tolist() == sorted(int(e) * I + j for e in ids for j in range(I))
    assert np.max(np.abs(y - dense)) < 1e-12


@both
def test_keep_zero_channels_is_shared_only(O):
    x, experts, sh, ids, w = _sparse_setup(10)
    kept, y = O.channel_select_token(x, ids, w, lambda e: experts[e],
                                     lambda e: O.down_norms(experts[e][2]), 0, shared=[sh])
    assert kept.size == 0
    assert np.max(np.abs(y - O.expert_output(x, *sh))) < 1e-15


@both
@pytest.mark.parametrize("mode", ["gate_dnorm", "router_weighted"])
@pytest.mark.parametrize("keep", [1, 2, 3, 4])
def test_channel_select_bruteforce(mode, keep, O):
    x, experts, sh, ids, w = _sparse_setup(11 + keep)
    I = experts[0][0].shape[0]
    cands = [(i, j) for i in range(len(ids)) for j in range(I)]

    def score(i, j):
        G, _, Dt = experts[ids[i]]
        g = sum(G[j][h] * x[h] for h in range(len(x)))
        s = abs(g / (1 + math.exp(-g))) * math.sqrt(sum(v * v for v in Dt[j]))
        return s * (w[i] if mode == "router_weighted" else 1.0)

    best = max(itertools.combinations(range(len(cands)), keep),
               key=lambda sub: sum(score(*cands[c]) for c in sub))
    kept, y = O.channel_select_token(x, ids, w, lambda e: experts[e],
                                     lambda e: O.down_norms(experts[e][2]), keep, mode=mode)
    assert kept.tolist() == sorted(int(ids[cands[c][0]]) * I + cands[c][1] for c in best)
    ref = [0.0] * len(x)
    for c in best:
        i, j = cands[c]
        G, V, Dt = experts[ids[i]]
        g = sum(G[j][h] * x[h] for h in range(len(x)))
        u = sum(V[j][h] * x[h] for h in range(len(x)))
        for h in range(len(x)):
            ref[h] += w[i] * g / (1 + math.exp(-g)) * u * Dt[j][h]
    assert np.max(np.abs(y - ref)) < 1e-12


@both
def test_equal_down_norms_rank_by_gate(O):
    rng = np.random.default_rng(12)
    H, I, E, k = 6, 8, 4, 2
    x = rng.normal(size=H)
    experts = []
    for _ in range(E):
        G, V, Dt = rand_expert(rng, I, H)
        Dt = Dt / np.linalg.norm(Dt, axis=1, keepdims=True)
        experts.append((G, V, Dt))
    ids, w = np.array([2, 0]), np.array([0.6, 0.4])
    kept, _ = O.channel_select_token(x, ids, w, lambda e: experts[e],
                                     lambda e: O.down_norms(experts[e][2]), 5)
    act = np.concatenate([np.abs(O.silu(experts[e][0] @ x)) for e in ids])
    cid = np.concatenate([e * I + np.arange(I) for e in ids])
    assert kept.tolist() == sorted(cid[np.argsort(-act, kind="stable")[:5]].tolist())


@both
def test_channel_ties_go_to_lower_channel_id(O):
    """Equal scores are kept in channel-id order e*I + j, not in routing-slot order: with the
    routing (1, 0) the four tied channels are, in slot order, ids 3, 4, 0, 1; the lowest
    three ids are 0, 1, 3."""
    H, I = 2, 3
    x = np.array([1.0, 0.0])
    G = np.array([[1.0, 0.0], [1.0, 0.0], [0.5, 0.0]])
    ex = (G, np.ones((I, H)), np.ones((I, H)))
    kept, _ = O.channel_select_token(x, np.array([1, 0]), np.array([0.5, 0.5]),
                                     lambda e: ex, lambda e: O.down_norms(ex[2]), 3)
    assert kept.tolist() == [0, 1, 3]


# ---------------------------------------------------------------- union and touched counts
@both
def test_union_matches_sets(O):
    rng = np.random.default_rng(13)
    E, k, B = 12, 3, 9
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)])
    n, touched, offsets, slots = O.union_experts(ids, E)
    assert touched.tolist() == sorted(set(ids.ravel().tolist()))
    assert n == len(touched)
    for e in range(E):
        want = [b * k + i for b in range(B) for i in range(k) if ids[b, i] == e]
        assert slots[offsets[e]:offsets[e + 1]].tolist() == want


@pytest.mark.parametrize("E,k,B", [(3, 1, 2), (4, 2, 2), (4, 1, 3), (5, 2, 2), (4, 3, 3)])
def test_expected_touched_exact_enumeration(E, k, B):
    closed = E * (1 - (1 - Fraction(k, E)) ** B)
    assert O.expected_touched_exact(E, k, B) == closed
    assert O.expected_touched(E, k, B) == pytest.approx(float(closed), rel=1e-14)


def test_expected_touched_pages_example():
    g = golden("touched_experts_e64_k3.json")
    E, k = g["E"], g["k"]
    for B, v in g["theory_column"].items():
        assert round(O.expected_touched(E, k, int(B)), 1) == v
    ex = g["worked_example"]
    assert round(1 - k / E, 3) == ex["p_not_chosen_by_one_token"]
    p_all = 1 - O.expected_touched(E, k, ex["B"]) / E
    assert round(p_all, 2) == ex["p_not_chosen_by_all"]
    assert round(1 - p_all, 2) == ex["p_used"]
    assert round(O.half_touched_batch(E, k), 1) == g["half_touched_batch"]


def test_touched_monte_carlo_uniform_routing():
    """Top-k of iid logits is a uniform k-subset; the mean union is the closed form."""
    rng = np.random.default_rng(14)
    E, k = 64, 3
    for B in (4, 16, 64):
        counts = []
        for _ in range(400):
            ids, _ = O.route(rng.normal(size=(B, E)), k)
            counts.append(O.union_experts(ids, E)[0])
        mu, sd = np.mean(counts), np.std(counts) / math.sqrt(len(counts))
        assert abs(mu - O.expected_touched(E, k, B)) < 4 * sd + 1e-9


# ---------------------------------------------------------------- bytes and ceilings
def test_bytes_formula_matches_table7_batch1():
    g = golden("table7_dram_reads.json")
    m = g["model"]
    b = O.layer_bytes(m["H"], m["I"], m["k"], "bf16")
    assert abs(b / 1e6 - g["full_model_mb_per_layer"]["1"]) < 0.15
    # batch 4 and 8: correlated routing reads less than the iid union bound
    for B in (4, 8):
        iid = O.layer_bytes(m["H"], m["I"], m["k"], "bf16",
                            n_experts_read=O.expected_touched(m["E"], m["k"], B))
        assert g["full_model_mb_per_layer"][str(B)] < iid / 1e6


def test_bytes_per_layer_of_the_stack_shapes():
    # 40-layer 256/8 bf16 stack with one shared expert: router + 8 routed + 1 shared
    b = O.layer_bytes(2048, 768, 8, "bf16", n_shared=1, I_shared=768, shared_dtype="bf16",
                      E=256, router_dtype="bf16")
    assert b == 1_048_576 + 75_497_472 + 9_437_184
    s = O.sparse_layer_bytes(2048, 768, 8, 799, "bf16", n_shared=1, I_shared=768, E=256,
                             router_dtype="bf16")
    assert s == 1_048_576 + 25_165_824 + 6_545_408 + 24_576 + 9_437_184
    assert O.layer_bytes(2048, 768, 8, "bf16", n_experts_read=0) == 0


def test_linear_expert_sizes_pages():
    g = golden("sparse501b_bytes.json")
    one = g["expert_side"] ** 2 * 2
    assert one == g["expert_bytes_mib"] * 2 ** 20
    assert round(one * g["experts"] / 1e9, 1) == g["all_experts_gb_printed"]
    assert g["total_params"] * 2 / 1e9 == g["bf16_total_gb"]
    assert g["active_params"] * 2 / 1e9 == g["bf16_active_gb"]
    assert g["total_params"] * 0.5 / 1e9 == pytest.approx(g["int4_total_gb"], rel=0.003)
    assert g["active_params"] * 0.5 / 1e9 == g["int4_active_gb"]


def test_decode_ceilings_pages():
    g = golden("moe_promise_ceilings.json")
    for mac, bw in g["achieved_gb_s"].items():
        c = O.decode_ceiling(bw, g["bytes_gb"]["35B-A3B-4bit"])
        assert round(c) == g["moe_ceilings_printed"][mac]
        frac = g["moe_measured_tok_s"][mac] / c
        lo, hi = g["moe_fraction_range_printed_percent"]
        assert lo - 0.5 <= 100 * frac <= hi + 0.5
    c = O.decode_ceiling(g["achieved_gb_s"]["office"], g["glm_744b_4bit_bytes_gb"])
    assert round(c) == g["glm_744b_ceiling_printed"]


def test_sector_billing_fig2c():
    g = golden("sector_billing.json")
    offs = [p[0] for p in g["pieces"]]
    lens = [p[1] for p in g["pieces"]]
    assert sum(lens) == g["needed_bytes"]
    assert O.billed_bytes(offs, lens, g["sector_bytes"]) == g["billed_bytes"]


# ---------------------------------------------------------------- linear experts
def test_linear_moe_matches_loops():
    rng = np.random.default_rng(15)
    E, k, B, Hin, Hout = 6, 2, 3, 5, 4
    M = [rng.normal(size=(Hout, Hin)) for _ in range(E)]
    X = rng.normal(size=(B, Hin))
    ids, w = O.route(rng.normal(size=(B, E)), k)
    Y = O.linear_moe(X, ids, w, lambda e: M[e])
    for b in range(B):
        for r in range(Hout):
            ref = sum(w[b, i] * sum(M[ids[b, i]][r][c] * X[b][c] for c in range(Hin))
                      for i in range(k))
            assert abs(Y[b, r] - ref) < 1e-12


# ---------------------------------------------------------------- generator (inputs)
def test_philox_known_answers():
    """Random123 known-answer vectors for Philox4x32-10."""
    import synth
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, out in kat:
        assert synth.philox4x32_10(ctr, key).tolist() == out


def test_generator_moments_and_subsets():
    import synth
    a = synth.normal_f32(0, 77, 0, 2_000_000, 0.02).astype(np.float64)
    assert abs(a.mean()) < 4 * 0.02 / math.sqrt(a.size)
    assert abs(a.std() / 0.02 - 1) < 0.005
    # any sub-range regenerates the same elements
    b = synth.normal_f32(0, 77, 1234, 100, 0.02)
    assert np.array_equal(b, a[1234:1334].astype(np.float32))
    c = synth.normal_bf16(0, 77, 1234, 100, 0.02)
    back = synth.bf16_bits_to_f32(c)
    assert np.all(np.abs(back - b) <= np.abs(b) * 2.0 ** -8)
