"""CPU oracle of the ternary-sketch channel screen.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP library never calls it.

Source: the jaehun.me review of arXiv:2610.37386, "The weights-only reader", stage 1 (the
sketch) and stage 2 (the output-unit score, eq. 1); the keep rule of "Background: channels and
keep rules".  What the method computes, in our notation:

* Load time, once per routed channel j: its gate row g_j and up row v_j are rotated in blocks
  of 128 coordinates by a randomized Hadamard transform R = H_128 diag(s) / sqrt(128) (s a
  fixed random sign vector per block; R is orthogonal, so g.x = (Rg).(Rx)).  Each rotated
  block is stored as ternary codes in {-1, 0, 1}, one FP16 scale, and rho_b, the block's mean
  squared quantization error.
* Per token: x is rotated once; per block only the 80 coordinates with the largest |Rx| are
  scanned, giving estimates g^_j ~ g_j.x and v^_j ~ v_j.x; the score is
  s_j = w_e ||d_j|| |silu(g^_j) v^_j| (eq. 1; without w_e in mode "gate_dnorm"); the K best
  channels over all of the token's routed experts are computed exactly from their full rows,
  the rest contribute nothing (their recovery, stage 3, is not part of this screen).

Readings where the pages leave a step open (each one is listed in the design notes):

* Work in the unnormalized rotated domain: u = H_128 (s * w) and z = H_128 (s * x) per block,
  so g.x = sum_b u_b.z_b / 128.  H_128 is the Sylvester-ordered Walsh-Hadamard matrix.
* Ternarization follows the ternary-weight-network rule (Li and Liu, 2016): threshold
  0.7 * mean|u| over the block, codes sign(u) where |u| exceeds it, scale = mean |u| over the
  nonzero codes (the squared-error optimum for those codes), stored as FP16 (round to
  nearest even); rho_b = mean over the block of (u - scale16 * code)^2, stored as FP16.
* The integer decisions (codes, and the 80 scanned coordinates) are taken in fp32 with the
  operation order of the GPU kernel, so both sides decide identically: the rotation as fp32
  butterflies, stage h = 1, 2, ..., 64, each (a + b, a - b) over pairs (i, i + h); block sums
  as fp32 trees (l + l^64, then l^32, ..., l^1 folds).  The estimates and scores themselves
  are computed in fp64 here.
* The 80 scanned coordinates of a block: the 80 largest |z|, ties to the lower coordinate.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import silu, to_f64, _row

BLOCK = 128
SCAN = 80


# ------------------------------------------------------------------ rotation (kernel order)
def fwht_f32(v: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform of each 128-block of the last axis, in fp32,
    butterfly stages h = 1, 2, ..., 64: (v[i], v[i+h]) -> (v[i] + v[i+h], v[i] - v[i+h])."""
    v = np.array(v, dtype=np.float32, copy=True)
    shp = v.shape
    v = v.reshape(-1, BLOCK)
    h = 1
    while h < BLOCK:
        w = v.reshape(v.shape[0], BLOCK // (2 * h), 2, h)
        a = w[:, :, 0, :].copy()
        b = w[:, :, 1, :].copy()
        w[:, :, 0, :] = a + b
        w[:, :, 1, :] = a - b
        v = w.reshape(-1, BLOCK)
        h *= 2
    return v.reshape(shp)


def rotate_f32(w: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """u = H_128 (s * w) per 128-block of the last axis (w widened to fp32 exactly; s = +-1)."""
    w = np.asarray(w, dtype=np.float32)
    s = np.asarray(signs, dtype=np.float32)
    return fwht_f32(w * s)


def hadamard_f64(n: int = BLOCK) -> np.ndarray:
    """The Sylvester Walsh-Hadamard matrix H_n (entries +-1), built by the doubling rule."""
    Hm = np.ones((1, 1))
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def tree_sum_f32(v: np.ndarray) -> np.float32:
    """Sum of 128 fp32 values in the kernel's order: a_l = v_l + v_{l+64} (l < 64), then
    a_l += a_{l^d} for d = 32, 16, 8, 4, 2, 1; returns a_0 (fp32 throughout)."""
    v = np.asarray(v, dtype=np.float32)
    a = (v[:64] + v[64:]).astype(np.float32)
    idx = np.arange(64)
    for d in (32, 16, 8, 4, 2, 1):
        a = (a + a[idx ^ d]).astype(np.float32)
    return np.float32(a[0])


# --------------------------------------------------------------------------- the sketch
def ternary_block(u: np.ndarray):
    """Codes, FP16 scale and FP16 rho of one rotated block u [128] (fp32)."""
    u = np.asarray(u, dtype=np.float32)
    au = np.abs(u).astype(np.float32)
    mean = np.float32(tree_sum_f32(au) * np.float32(1.0 / BLOCK))
    thr = np.float32(np.float32(0.7) * mean)
    code = np.where(au > thr, np.sign(u), 0).astype(np.int8)
    nnz = int(np.count_nonzero(code))
    if nnz:
        alpha = np.float32(tree_sum_f32(np.where(code != 0, au, np.float32(0))) /
                           np.float32(nnz))
    else:
        alpha = np.float32(0)
    a16 = np.float16(alpha)
    err = (u - np.float32(a16) * code.astype(np.float32)).astype(np.float32)
    rho = np.float16(np.float32(tree_sum_f32(err * err) * np.float32(1.0 / BLOCK)))
    return code, a16, rho


def sketch_rows(W, signs):
    """The sketch of a stored [rows][H] tensor: codes int8 [rows][H] in {-1,0,1} (rotated
    coordinates), alpha float16 [rows][H/128], rho float16 [rows][H/128]."""
    Wf = np.asarray(to_f64(W), dtype=np.float32)  # bf16 / fp32 storage widen exactly
    U = rotate_f32(Wf, signs)
    R, H = U.shape
    nb = H // BLOCK
    codes = np.empty((R, H), dtype=np.int8)
    alpha = np.empty((R, nb), dtype=np.float16)
    rho = np.empty((R, nb), dtype=np.float16)
    for r in range(R):
        for b in range(nb):
            c, a, p = ternary_block(U[r, b * BLOCK:(b + 1) * BLOCK])
            codes[r, b * BLOCK:(b + 1) * BLOCK] = c
            alpha[r, b] = a
            rho[r, b] = p
    return codes, alpha, rho


# ----------------------------------------------------------------------- the token side
def scan_mask(z: np.ndarray, n: int = SCAN) -> np.ndarray:
    """Per 128-block of z [H], the n coordinates of largest |z| (ties to the lower
    coordinate) as a boolean mask [H]."""
    z = np.asarray(z, dtype=np.float32)
    H = z.shape[0]
    m = np.zeros(H, dtype=bool)
    for b in range(H // BLOCK):
        a = np.abs(z[b * BLOCK:(b + 1) * BLOCK])
        order = np.lexsort((np.arange(BLOCK), -a.astype(np.float64)))[:n]
        m[b * BLOCK + order] = True
    return m


def estimate(codes, alpha, z, mask) -> np.ndarray:
    """Sketch estimates of the rows' dot products with x: sum over blocks b of
    alpha_b * sum over the scanned coordinates i of code_i z_i, divided by 128 (fp64)."""
    codes = np.atleast_2d(codes).astype(np.float64)
    alpha = np.atleast_2d(alpha).astype(np.float64)
    zz = np.where(mask, np.asarray(z, dtype=np.float64), 0.0)
    R, H = codes.shape
    nb = H // BLOCK
    per_block = (codes * zz[None, :]).reshape(R, nb, BLOCK).sum(axis=2)
    return (alpha * per_block).sum(axis=1) / BLOCK


def sketch_scores(x, ids, w, sketch_of, dnorm_of, signs, mode="router_weighted", scan=SCAN):
    """Eq. 1 scores [k][I] of the token's candidates, with the estimates g^, v^ [k][I]."""
    z = rotate_f32(np.asarray(x, dtype=np.float32), signs)
    m = scan_mask(z, scan)
    ss, gs, vs = [], [], []
    for e, we in zip(ids, w):
        (gc, ga, _), (vc, va, _) = sketch_of(int(e))
        gh = estimate(gc, ga, z, m)
        vh = estimate(vc, va, z, m)
        s = np.abs(silu(gh) * vh) * dnorm_of(int(e))
        if mode == "router_weighted":
            s = we * s
        elif mode != "gate_dnorm":
            raise ValueError(mode)
        ss.append(s)
        gs.append(gh)
        vs.append(vh)
    return np.stack(ss), np.stack(gs), np.stack(vs)


def sketch_select_token(x, ids, w, get_expert, sketch_of, dnorm_of, keep, signs, shared=(),
                        mode="router_weighted", scan=SCAN):
    """The screened layer for one token: rank the k*I candidates by the sketch scores (ties to
    the lower e*I + j), compute the first `keep` exactly from their full gate, up and down
    rows, add the shared experts.  Returns (kept ids e*I + j ascending [keep], y [H])."""
    x64 = np.asarray(x, dtype=np.float64).reshape(-1)
    s, _, _ = sketch_scores(x, ids, w, sketch_of, dnorm_of, signs, mode, scan)
    k, I = s.shape
    cid = (np.asarray(ids, dtype=np.int64)[:, None] * I + np.arange(I)[None, :]).reshape(-1)
    order = np.lexsort((cid, -s.reshape(-1)))[:keep]
    y = np.zeros_like(x64)
    for f in order:
        i, j = divmod(int(f), I)
        G, V, Dt = get_expert(int(ids[i]))
        g = float(to_f64(_row(G, j)).reshape(-1) @ x64)
        u = float(to_f64(_row(V, j)).reshape(-1) @ x64)
        y += w[i] * (silu(g) * u) * to_f64(_row(Dt, j)).reshape(-1)
    for (gs_, us_, ds_) in shared:
        gx = to_f64(gs_) @ x64
        y += to_f64(ds_).T @ (silu(gx) * (to_f64(us_) @ x64))
    return np.sort(cid[order]), y


# ------------------------------------------------------------------ stage 3: recovery
RANK = 32


def recovery_basis(down_rows_iter, H, rank=RANK):
    """U [H][rank]: the top-`rank` left singular vectors of the layer's stacked down columns
    d_j (every routed channel of every expert), as eigenvectors of sum_j d_j d_j^T (fp64),
    largest eigenvalue first; each column's sign fixed so that its largest-magnitude entry is
    positive.  `down_rows_iter` yields [rows][H] blocks of d_j (any storage form)."""
    G = np.zeros((H, H), dtype=np.float64)
    for blk in down_rows_iter:
        D = to_f64(blk).reshape(-1, H)
        G += D.T @ D
    vals, vecs = np.linalg.eigh(G)
    U = vecs[:, ::-1][:, :rank].copy()
    for c in range(U.shape[1]):
        i = int(np.argmax(np.abs(U[:, c])))
        if U[i, c] < 0:
            U[:, c] = -U[:, c]
    return U


def recovery_coeffs(down_t, U):
    """b_j = U^T d_j for the rows of one expert's D^T [I][H] -> [I][rank] (fp64)."""
    return to_f64(down_t).reshape(-1, U.shape[0]) @ U


def reader_token(x, ids, w, get_expert, sketch_of, dnorm_of, keep, signs, U, coeffs_of,
                 shared=(), mode="router_weighted", scan=SCAN, p_exact=False):
    """The reader for one token (stages 1-3, eq. 2): the screen of sketch_select_token, then
    the dropped channels S added through the rank-r map: y^ = sum_K w_j d_j a_j
    + U sum_S w_j b_j p_j, with p_j = silu(g^_j) v^_j the screen's own activation estimates
    (p_exact: the exact a_j instead, for pins).  coeffs_of(e) -> b [I][rank] of expert e.
    Returns (kept ids ascending, y [H])."""
    x64 = np.asarray(x, dtype=np.float64).reshape(-1)
    kept, y = sketch_select_token(x, ids, w, get_expert, sketch_of, dnorm_of, keep, signs,
                                  shared, mode, scan)
    _, gh, vh = sketch_scores(x, ids, w, sketch_of, dnorm_of, signs, mode, scan)
    k, I = gh.shape
    keptset = set(int(c) for c in kept)
    r = np.zeros(U.shape[1], dtype=np.float64)
    for i, e in enumerate(ids):
        b = coeffs_of(int(e))
        for j in range(I):
            if int(e) * I + j in keptset:
                continue
            if p_exact:
                G, V, _ = get_expert(int(e))
                p = silu(float(to_f64(_row(G, j)).reshape(-1) @ x64)) * \
                    float(to_f64(_row(V, j)).reshape(-1) @ x64)
            else:
                p = silu(gh[i, j]) * vh[i, j]
            r += w[i] * p * b[j]
    return kept, y + U @ r


def sketch_bytes(H, I, k, keep, b_e=2.0, scan=SCAN):
    """Bytes one token reads in the screen of one layer's routed experts: the sketch of every
    candidate's gate and up rows (2-bit codes, all coordinates of a block lie in its 32 code
    bytes, and FP16 scales), then the kept channels' full gate, up and down rows."""
    nb = H // BLOCK
    sketch = k * I * 2 * nb * (BLOCK // 4 + 2)
    return sketch + 3 * keep * H * b_e
