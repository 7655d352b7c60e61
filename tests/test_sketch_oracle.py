"""Pins of the ternary-sketch screen's oracle (CPU only): the rotation against the Hadamard
matrix and its orthogonality, rows that are exactly ternary in the rotated basis giving exact
sketches and exact estimates, the full scan, the squared-error optimality of the scale, rho's
definition, the scanned-coordinate rule with ties, and the keep rule by brute force.

Source: the jaehun.me review of arXiv:2610.37386, "The weights-only reader", stages 1 and 2."""
import itertools
import math

import numpy as np
import pytest

from oracle import sketch_oracle as S

B = S.BLOCK


def _signs(rng, H):
    return np.where(rng.normal(size=H) < 0, -1, 1).astype(np.int8)


def test_hadamard_builder_is_orthogonal_up_to_n():
    Hm = S.hadamard_f64()
    assert Hm.shape == (B, B)
    assert np.array_equal(Hm @ Hm.T, B * np.eye(B))
    assert set(np.unique(Hm)) == {-1.0, 1.0}


def test_fwht_matches_the_matrix_product():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(4, 3 * B)).astype(np.float32)
    Hm = S.hadamard_f64()
    ref = np.concatenate([v[:, b * B:(b + 1) * B].astype(np.float64) @ Hm.T for b in range(3)],
                         axis=1)
    got = S.fwht_f32(v).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 8 * np.finfo(np.float32).eps * np.max(np.abs(ref))
    # exact for small integers (no rounding in any butterfly)
    iv = rng.integers(-8, 9, size=(2, B)).astype(np.float32)
    assert np.array_equal(S.fwht_f32(iv).astype(np.float64), iv.astype(np.float64) @ Hm.T)


def test_rotation_preserves_dot_products():
    """g.x = (R g).(R x) with R = H diag(s) / sqrt(128): in the unnormalized domain,
    u.z / 128."""
    rng = np.random.default_rng(2)
    H = 2 * B
    g, x = rng.normal(size=H), rng.normal(size=H)
    s = _signs(rng, H)
    Hm = S.hadamard_f64()
    u = np.concatenate([Hm @ (s[b * B:(b + 1) * B] * g[b * B:(b + 1) * B]) for b in range(2)])
    z = np.concatenate([Hm @ (s[b * B:(b + 1) * B] * x[b * B:(b + 1) * B]) for b in range(2)])
    assert abs(u @ z / B - g @ x) < 1e-12 * (np.abs(g) @ np.abs(x))


def _exactly_ternary_rows(rng, rows, H, s):
    """Rows whose rotated blocks are exactly alpha_b * c (alpha a power of two, c ternary)."""
    c = rng.choice([-1, 0, 1], size=(rows, H), p=[0.35, 0.3, 0.35]).astype(np.int8)
    alpha = 2.0 ** rng.integers(-6, -2, size=(rows, H // B))
    u = c * np.repeat(alpha, B, axis=1)
    Hm = S.hadamard_f64()
    g = np.concatenate([(Hm @ u[:, b * B:(b + 1) * B].T).T for b in range(H // B)], axis=1)
    g = g * s.astype(np.float64) / B          # R^T u in the unnormalized convention
    return g, c, alpha


def test_exactly_ternary_rows_give_exact_sketch_and_estimates():
    rng = np.random.default_rng(3)
    H = 2 * B
    s = _signs(rng, H)
    g, c, alpha = _exactly_ternary_rows(rng, 5, H, s)
    assert np.array_equal(g.astype(np.float32).astype(np.float64), g)   # exact in fp32
    codes, a16, rho = S.sketch_rows(g, s)
    assert np.array_equal(codes, c)
    assert np.array_equal(a16.astype(np.float64), alpha)
    assert np.all(rho == 0)
    x = rng.normal(size=H).astype(np.float32)
    z = S.rotate_f32(x, s)
    full = np.ones(H, dtype=bool)
    est = S.estimate(codes, a16, z, full)
    ref = g @ x.astype(np.float64)
    assert np.max(np.abs(est - ref)) < 1e-5 * np.max(np.abs(ref))  # z carries fp32 rounding


def test_full_scan_is_the_whole_sketch_dot_product():
    rng = np.random.default_rng(4)
    H = 3 * B
    s = _signs(rng, H)
    W = rng.normal(0, 0.02, size=(4, H))
    codes, a16, _ = S.sketch_rows(W, s)
    z = S.rotate_f32(rng.normal(size=H), s).astype(np.float64)
    m = S.scan_mask(z, B)
    assert m.all()
    ref = [sum(float(a16[r, b]) * float(codes[r, b * B:(b + 1) * B] @ z[b * B:(b + 1) * B])
               for b in range(H // B)) / B for r in range(4)]
    assert np.allclose(S.estimate(codes, a16, z, m), ref, rtol=1e-12, atol=0)


def test_scale_is_the_squared_error_optimum_and_rho_is_the_mean_squared_error():
    rng = np.random.default_rng(5)
    for _ in range(20):
        u = rng.normal(size=B).astype(np.float32)
        c, a16, rho = S.ternary_block(u)
        # threshold rule: codes are sign(u) exactly where |u| > 0.7 mean|u|
        thr = 0.7 * np.mean(np.abs(u.astype(np.float64)))
        far = np.abs(np.abs(u) - thr) > 1e-5
        assert np.array_equal((c != 0)[far], (np.abs(u) > thr)[far])
        assert np.all(c[c != 0] == np.sign(u[c != 0]))
        # the scale minimises sum (u - a c)^2 for these codes: a* = sum|u| over nonzero / nnz
        nz = c != 0
        a_star = np.abs(u[nz].astype(np.float64)).mean()
        assert abs(float(a16) - a_star) <= 2 ** -10 * a_star      # FP16 rounding
        mse = lambda a: np.mean((u.astype(np.float64) - a * c) ** 2)
        assert mse(a_star) <= min(mse(a_star * 1.01), mse(a_star * 0.99))
        # rho: the block's mean squared error with the stored scale (FP16)
        ref = mse(float(a16))
        assert abs(float(rho) - ref) <= 2 ** -10 * ref + 1e-7


def test_scan_mask_takes_the_largest_with_ties_to_the_lower_coordinate():
    z = np.zeros(B, dtype=np.float32)
    z[:10] = np.arange(10, 0, -1)          # 10 .. 1
    z[10:20] = 5.0                          # ties with z[5]
    z[20:] = -0.5
    m = S.scan_mask(z, 12)
    want = list(range(5)) + [5] + list(range(10, 16))   # 10..6, then the 5.0s in index order
    assert np.nonzero(m)[0].tolist() == sorted(want)
    rng = np.random.default_rng(6)
    z = rng.normal(size=2 * B).astype(np.float32)
    m = S.scan_mask(z, S.SCAN)
    for b in range(2):
        blk = np.abs(z[b * B:(b + 1) * B])
        chosen = m[b * B:(b + 1) * B]
        assert chosen.sum() == S.SCAN
        assert blk[chosen].min() >= blk[~chosen].max()


@pytest.mark.parametrize("mode", ["gate_dnorm", "router_weighted"])
def test_screen_keep_rule_bruteforce(mode):
    """The screened layer keeps the `keep` candidates of largest eq.-1 score (brute force over
    all subsets) and computes them from their full rows."""
    rng = np.random.default_rng(7 if mode == "gate_dnorm" else 8)
    H, I, E = B, 3, 4
    s = _signs(rng, H)
    experts = [tuple(rng.normal(0, 0.3, size=(I, H)) for _ in range(3)) for _ in range(E)]
    sk = {e: (S.sketch_rows(experts[e][0], s), S.sketch_rows(experts[e][1], s))
          for e in range(E)}
    sketch_of = lambda e: ((sk[e][0][0], sk[e][0][1], None), (sk[e][1][0], sk[e][1][1], None))
    dn = {e: np.linalg.norm(experts[e][2], axis=1) for e in range(E)}
    ids, w = np.array([2, 0]), np.array([0.7, 0.3])
    x = rng.normal(size=H)
    sc, gh, vh = S.sketch_scores(x, ids, w, sketch_of, dn.__getitem__, s, mode)
    for keep in (1, 2, 4):
        cands = [(i, j) for i in range(2) for j in range(I)]
        best = max(itertools.combinations(range(len(cands)), keep),
                   key=lambda sub: sum(sc[cands[q]] for q in sub))
        kept, y = S.sketch_select_token(x, ids, w, lambda e: experts[e], sketch_of,
                                        dn.__getitem__, keep, s, mode=mode)
        assert kept.tolist() == sorted(int(ids[cands[q][0]]) * I + cands[q][1] for q in best)
        ref = np.zeros(H)
        for q in best:
            i, j = cands[q]
            G, V, Dt = experts[ids[i]]
            g, u = G[j] @ x, V[j] @ x
            ref += w[i] * g / (1 + math.exp(-g)) * u * Dt[j]
        assert np.max(np.abs(y - ref)) < 1e-12


def test_sketch_scores_follow_eq1():
    rng = np.random.default_rng(9)
    H, I = 2 * B, 5
    s = _signs(rng, H)
    G, V = rng.normal(0, 0.1, size=(I, H)), rng.normal(0, 0.1, size=(I, H))
    gk, vk = S.sketch_rows(G, s), S.sketch_rows(V, s)
    x = rng.normal(size=H)
    dn = np.abs(rng.normal(size=I)) + 0.5
    sc, gh, vh = S.sketch_scores(x, [3], [0.25], lambda e: (gk, vk), lambda e: dn, s)
    z = S.rotate_f32(x, s)
    m = S.scan_mask(z)
    g_ref = S.estimate(gk[0], gk[1], z, m)
    v_ref = S.estimate(vk[0], vk[1], z, m)
    assert np.allclose(gh[0], g_ref) and np.allclose(vh[0], v_ref)
    assert np.allclose(sc[0], 0.25 * dn * np.abs(g_ref / (1 + np.exp(-g_ref)) * v_ref),
                       rtol=1e-14)


def test_sketch_bytes_arithmetic():
    # per candidate: 2 rows x 16 blocks x (32 code bytes + 2 scale bytes); kept: 3 full rows
    assert S.sketch_bytes(2048, 768, 8, 799) == 8 * 768 * 2 * 16 * 34 + 3 * 799 * 4096


# ------------------------------------------------------------------ stage 3: recovery
def _tiny_reader(rng, H=B, E=3, I=4):
    s = _signs(rng, H)
    experts = [tuple(rng.normal(0, 0.3, size=(I, H)) for _ in range(3)) for _ in range(E)]
    sk = {e: (S.sketch_rows(experts[e][0], s), S.sketch_rows(experts[e][1], s))
          for e in range(E)}
    sketch_of = lambda e: sk[e]
    dn = {e: np.linalg.norm(experts[e][2], axis=1) for e in range(E)}
    return s, experts, sketch_of, dn


def test_full_rank_map_with_exact_activations_is_the_dense_layer():
    """Rank H with p = a: the recovery adds back every dropped channel exactly, so the output
    is the dense layer's for any keep."""
    rng = np.random.default_rng(21)
    s, experts, sketch_of, dn = _tiny_reader(rng)
    U = np.linalg.qr(rng.normal(size=(B, B)))[0]          # any orthonormal basis of R^H
    coeffs = {e: S.recovery_coeffs(experts[e][2], U) for e in range(3)}
    ids, w = np.array([2, 0]), np.array([0.7, 0.3])
    x = rng.normal(size=B)
    from oracle import moe_oracle as O
    dense = O.moe_layer_given(x, ids, w, lambda e: experts[e])
    for keep in (0, 1, 5, 8):
        _, y = S.reader_token(x, ids, w, lambda e: experts[e], sketch_of, dn.__getitem__, keep,
                              s, U, coeffs.__getitem__, p_exact=True)
        assert np.allclose(y, dense, rtol=0, atol=1e-10 * np.max(np.abs(dense)))


def test_keep_all_adds_nothing_and_keep_none_is_the_map_alone():
    rng = np.random.default_rng(22)
    s, experts, sketch_of, dn = _tiny_reader(rng)
    U = np.linalg.qr(rng.normal(size=(B, 8)))[0]
    coeffs = {e: S.recovery_coeffs(experts[e][2], U) for e in range(3)}
    ids, w = np.array([1, 2]), np.array([0.4, 0.6])
    x = rng.normal(size=B)
    kept, y = S.reader_token(x, ids, w, lambda e: experts[e], sketch_of, dn.__getitem__, 8, s,
                             U, coeffs.__getitem__)
    _, y_screen = S.sketch_select_token(x, ids, w, lambda e: experts[e], sketch_of,
                                        dn.__getitem__, 8, s)
    assert kept.size == 8 and np.allclose(y, y_screen, rtol=0, atol=1e-12)
    # keep 0: y = U sum_all w b p with the screen's estimates
    _, gh, vh = S.sketch_scores(x, ids, w, sketch_of, dn.__getitem__, s)
    r = sum(w[i] * (gh[i, j] / (1 + np.exp(-gh[i, j]))) * vh[i, j] * coeffs[int(e)][j]
            for i, e in enumerate(ids) for j in range(4))
    _, y0 = S.reader_token(x, ids, w, lambda e: experts[e], sketch_of, dn.__getitem__, 0, s,
                           U, coeffs.__getitem__)
    assert np.allclose(y0, U @ r, rtol=0, atol=1e-12)


def test_recovery_basis_is_the_top_singular_subspace():
    rng = np.random.default_rng(23)
    H = 16
    D = rng.normal(size=(40, H)) @ np.diag(np.linspace(3.0, 0.1, H))   # distinct spectrum
    U = S.recovery_basis([D[:17], D[17:]], H, rank=5)
    assert np.allclose(U.T @ U, np.eye(5), atol=1e-12)
    Us = np.linalg.svd(D.T, full_matrices=False)[0][:, :5]
    assert np.allclose(U @ U.T, Us @ Us.T, atol=1e-10)     # the same subspace
    for c in range(5):
        assert U[np.argmax(np.abs(U[:, c])), c] > 0
