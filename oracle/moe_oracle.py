"""CPU oracle for the routed-expert FFN layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its binding)
never calls it and must fail if its native library is missing.

Plain numpy in float64: every weight and activation is widened exactly from its storage
type (fp32, bf16 or MXFP4) and every sum is a float64 library product or sum.  No blocking,
fusion or reordering beyond what the definitions state.  Sources (web pages; cited by page
title and section):

* [MoE-arith]  "Mixture of Experts Changes the Arithmetic" (creativeworksofknowledge.com),
  sections "Two Numbers Instead of One" and "What the Runtime Does With the Promise".
* [Reader]     the jaehun.me review of arXiv:2610.37386 (weights-only channel reader),
  sections "Background: channels and keep rules" (Fig. 2), "The weights-only reader"
  stage 2 (eq. 1), Table 3 and Table 7.
* [Sparse-501B] "501B of which 23B are switched on: the arithmetic of 4.6%"
  (blog.mna-game...), section 2 "Core concepts" and section 3 [B].

Readings where the pages are silent (each is listed with its reason in the design notes):
the gate nonlinearity phi is silu; the router weights are a softmax over the k selected
logits; ties in a top-k go to the lower index; shared experts have weight 1 and are never
channel-selection candidates; MXFP4 follows the OCP Microscaling v1.0 e2m1/e8m0 format.
"""
from __future__ import annotations

import math
from fractions import Fraction
from itertools import combinations, product

import numpy as np

# ----------------------------------------------------------------------------------------
# Storage decoding (exact widening to float64)
# ----------------------------------------------------------------------------------------

# e2m1 magnitudes of codes 0..7 (OCP Microscaling Formats v1.0, FP4 E2M1 element format).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
        .astype(np.float64)


def mxfp4_to_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64 (exact).

    codes [rows, cols/2] uint8 (even element in the low nibble), scales [rows, cols/32]
    e8m0 bytes.  value = (-1)^s * e2m1(code) * 2^(scale - 127).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    nib = np.empty((rows, codes.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    mag = E2M1_MAGNITUDES[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    exps = np.asarray(scales, dtype=np.int64) - 127
    return val * np.repeat(np.ldexp(1.0, exps), 32, axis=1)


def to_f64(t) -> np.ndarray:
    """Widen a stored tensor: float32/float64 arrays, ('bf16', u16) or ('mxfp4', codes, scales)."""
    if isinstance(t, tuple):
        if t[0] == "bf16":
            return bf16_to_f64(t[1])
        if t[0] == "mxfp4":
            return mxfp4_to_f64(t[1], t[2])
        raise ValueError(t[0])
    return np.asarray(t, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# Routing: router logits, top-k, softmax weights
# ----------------------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router) -> np.ndarray:
    """l = W_r x, one score per expert [Reader, "Background"; MoE-arith, "Two Numbers"].

    x [B, H] (or [H]); W_r [E, H].  Returns float64 [B, E].
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ to_f64(w_router).T


def topk_order(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, largest first, ties to the lower index."""
    scores = np.asarray(scores, dtype=np.float64)
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -scores))  # primary: score descending; secondary: index
    return order[:k]


def softmax_selected(sel_logits: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits only (renormalised top-k gate)."""
    m = np.max(sel_logits)
    e = np.exp(sel_logits - m)
    return e / np.sum(e)


def route(logits: np.ndarray, k: int):
    """Top-k experts per token in routing order and their softmax weights.

    Each token picks k of E experts, re-chosen in every layer [MoE-arith, "Two Numbers"].
    Returns ids [B, k] int64 (descending logit, ties to the lower id) and w [B, k] float64.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    B = logits.shape[0]
    ids = np.empty((B, k), dtype=np.int64)
    w = np.empty((B, k), dtype=np.float64)
    for b in range(B):
        ids[b] = topk_order(logits[b], k)
        w[b] = softmax_selected(logits[b, ids[b]])
    return ids, w


def topk_margin(logits_row: np.ndarray, k: int) -> float:
    """Smallest gap among the k+1 largest logits (fixes both the selected set and its order)."""
    s = np.sort(np.asarray(logits_row, dtype=np.float64))[::-1][: k + 1]
    if s.shape[0] < 2:
        return math.inf
    return float(np.min(s[:-1] - s[1:]))


# ----------------------------------------------------------------------------------------
# The gated-MLP expert, channel by channel
# ----------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_activations(x: np.ndarray, gate, up) -> np.ndarray:
    """a_j = phi(g_j . x) (v_j . x) for every channel j [Reader, "Background"].

    Channel j owns row j of G_e and row j of V_e.  x [H]; G, V [I, H].  Returns [I].
    """
    x = np.asarray(x, dtype=np.float64)
    g = to_f64(gate) @ x
    u = to_f64(up) @ x
    return silu(g) * u


def expert_output(x: np.ndarray, gate, up, down_t) -> np.ndarray:
    """sum_j a_j d_j, where d_j is column j of D_e, stored as row j of D_e^T [I, H]."""
    a = expert_activations(x, gate, up)
    return to_f64(down_t).T @ a


def moe_layer_token(x, w_router, get_expert, k, shared=(), logits=None):
    """One token through the routed expert FFN layer (B = 1).

    y = sum over the k routed experts e of w_e * sum_j a_j d_j
        + sum over shared experts s of sum_j a_j d_j
    Routed output is the router-weighted sum of a_j d_j [Reader, "Background"]; shared
    experts are read by every token [MoE-arith, "Two Numbers"], with weight 1.

    get_expert(e) -> (G_e, V_e, D_e^T); shared: sequence of (G, V, D^T).
    Returns (y [H] float64, ids [k], w [k]).
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    if logits is None:
        logits = router_logits(x, w_router)[0]
    ids, w = route(np.asarray(logits)[None, :], k)
    ids, w = ids[0], w[0]
    y = np.zeros_like(x)
    for e, we in zip(ids, w):
        y += we * expert_output(x, *get_expert(int(e)))
    for (g, u, d) in shared:
        y += expert_output(x, g, u, d)
    return y, ids, w


def moe_layer_given(x, ids, w, get_expert, shared=()):
    """The same layer output for a routing given as ids [k'] and weights w [k']: the
    router-weighted sum of the listed experts' outputs plus the shared experts
    [Reader, "Background"; MoE-arith, "Two Numbers"]."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    y = np.zeros_like(x)
    for e, we in zip(ids, w):
        y += float(we) * expert_output(x, *get_expert(int(e)))
    for (g, u, d) in shared:
        y += expert_output(x, g, u, d)
    return y


# ----------------------------------------------------------------------------------------
# Channel-sparse variant: fixed-count top-K keep rule across all routed experts
# ----------------------------------------------------------------------------------------

def down_norms(down_t) -> np.ndarray:
    """||d_j||_2 per channel, computed once at load [Reader, "The weights-only reader", stage 2]."""
    d = to_f64(down_t)
    return np.sqrt(np.sum(d * d, axis=-1))


def channel_scores(x, ids, w, get_expert, dnorm_of, mode="gate_dnorm"):
    """Score of every candidate channel (e, j) of the token's routed experts.

    gate_dnorm:       s = |silu(g_j . x)| * ||d_j||
    router_weighted:  s = w_e * |silu(g_j . x)| * ||d_j||   (the output units of eq. 1,
                      with the exact gate in place of the sketch estimate)
    The output-unit score lets channels of different experts be compared directly, so the
    keep set is chosen across all of the token's experts [Reader, stage 2, eq. 1].
    Returns scores [k, I] and gate values g [k, I].
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    gs, ss = [], []
    for e, we in zip(ids, w):
        G, _, _ = get_expert(int(e))
        g = to_f64(G) @ x
        s = np.abs(silu(g)) * dnorm_of(int(e))
        if mode == "router_weighted":
            s = we * s
        elif mode != "gate_dnorm":
            raise ValueError(mode)
        gs.append(g)
        ss.append(s)
    return np.stack(ss), np.stack(gs)


def channel_select_token(x, ids, w, get_expert, dnorm_of, keep, shared=(),
                         mode="gate_dnorm"):
    """Fixed-count top-K keep rule over the k*I candidates of one token.

    Kept channels are computed exactly from their full rows; dropped channels contribute
    nothing and their up rows and down columns are never read [Reader, "Background"].  A
    channel is row j of expert e, identified by e*I + j [Reader, "Background": channel j owns
    row j of G_e and V_e and column j of D_e].  Candidates are ranked by score, ties to the
    lower e*I + j; the first `keep` are kept.  Returns (kept channel ids e*I + j ascending
    [K], y [H]).
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    s, g = channel_scores(x, ids, w, get_expert, dnorm_of, mode)
    k, I = s.shape
    cid = (np.asarray(ids, dtype=np.int64)[:, None] * I + np.arange(I)[None, :]).reshape(-1)
    order = np.lexsort((cid, -s.reshape(-1)))[:keep]  # score descending, then channel id
    y = np.zeros_like(x)
    for f in order:
        i, j = divmod(int(f), I)
        _, V, Dt = get_expert(int(ids[i]))
        vj = to_f64(_row(V, j))
        dj = to_f64(_row(Dt, j))
        a = silu(g[i, j]) * float(vj.reshape(-1) @ x)
        y += w[i] * a * dj.reshape(-1)
    for (gs, us, ds) in shared:
        y += expert_output(x, gs, us, ds)
    return np.sort(cid[order]), y


def channel_select_threshold_token(x, ids, w, get_expert, dnorm_of, tau, shared=(),
                                   mode="gate_dnorm"):
    """Threshold keep rule over the k*I candidates of one token [Reader, "Background: channels
    and keep rules", the first row of its table: every channel whose score is at least tau
    passes, so the number kept -- and the bytes read -- change from token to token].  The same
    scores and the same exact computation of the kept channels as channel_select_token.
    Returns (kept channel ids e*I + j ascending, y [H])."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    s, g = channel_scores(x, ids, w, get_expert, dnorm_of, mode)
    k, I = s.shape
    cid = (np.asarray(ids, dtype=np.int64)[:, None] * I + np.arange(I)[None, :]).reshape(-1)
    keep = np.nonzero(s.reshape(-1) >= tau)[0]
    y = np.zeros_like(x)
    for f in keep:
        i, j = divmod(int(f), I)
        _, V, Dt = get_expert(int(ids[i]))
        a = silu(g[i, j]) * float(to_f64(_row(V, j)).reshape(-1) @ x)
        y += w[i] * a * to_f64(_row(Dt, j)).reshape(-1)
    for (gs, us, ds) in shared:
        y += expert_output(x, gs, us, ds)
    return np.sort(cid[keep]), y


def batch_channel_scores(X, ids, w, get_expert, dnorm_of):
    """The batch scores of batch-wide channel selection [Reader, "Limits"; the score is the
    router-weighted output-unit score of "Background: channels and keep rules", summed over
    the batch].  Reading taken: the candidates are the channels (e, j) of the experts any
    token of the batch routes to, in ascending e*I + j; a channel's batch score is the sum over
    the tokens b routed to e of w_{b,e} ||d_j|| |silu(g_j.x_b)|.  Returns (candidate ids e*I + j,
    their scores, the activations {(e, b): (w_{b,e}, silu(g.x_b) * (v.x_b) over the channels)})."""
    X = np.asarray(X, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    B = ids.shape[0]
    touched = sorted(set(int(e) for e in ids.ravel()))
    cids, svals, acts = [], [], {}
    for e in touched:
        G, V, _ = get_expert(e)
        Gm, Vm = to_f64(G), to_f64(V)
        I = Gm.shape[0]
        dn = np.asarray(dnorm_of(e), dtype=np.float64)
        sc = np.zeros(I)
        for b in range(B):
            hit = np.nonzero(ids[b] == e)[0]
            if hit.size == 0:
                continue
            wb = w[b, hit[0]]
            g = Gm @ X[b]
            sc += wb * dn * np.abs(silu(g))
            acts[(e, b)] = (wb, silu(g) * (Vm @ X[b]))
        cids.append(e * I + np.arange(I))
        svals.append(sc)
    if not touched:
        return np.zeros(0, dtype=np.int64), np.zeros(0), acts
    return np.concatenate(cids), np.concatenate(svals), acts


def batch_channel_select(X, ids, w, get_expert, dnorm_of, keep, shared=()):
    """Batch-wide channel selection for B tokens [Reader, "Limits": selecting the whole
    batch's channels at once is the authors' future work; Table 7 measures the per-token
    reader at B = 4 and 8].  Reading taken: the candidates and batch scores of
    batch_channel_scores; the `keep` best batch scores are kept (ties to the lower e*I + j),
    and each kept channel is computed exactly for every token routed to its expert (its rows
    read once for the batch); dropped channels contribute nothing; shared experts are computed
    in full for every token.  Returns (kept ids e*I + j ascending, Y [B][H])."""
    X = np.asarray(X, dtype=np.float64)
    B = X.shape[0]
    cid, sv, acts = batch_channel_scores(X, ids, w, get_expert, dnorm_of)
    order = np.lexsort((cid, -sv))[:keep]
    kept = np.sort(cid[order])
    Y = np.zeros_like(X)
    I = acts[next(iter(acts))][1].size if acts else 1
    for c in kept:
        e, j = divmod(int(c), I)
        dj = to_f64(_row(get_expert(e)[2], j)).reshape(-1)
        for b in range(B):
            if (e, b) in acts:
                wb, a = acts[(e, b)]
                Y[b] += wb * a[j] * dj
    for b in range(B):
        for (gs, us, ds) in shared:
            Y[b] += expert_output(X[b], gs, us, ds)
    return kept, Y


def calibrate_tau(score_sets, frac):
    """The threshold calibrated on a set of tokens [Reader, calibration discussion: tau is set
    on calibration data so that the kept fraction meets the budget on average]: the m-th
    largest of the pooled scores of all calibration tokens, m = round(frac * total) (half up),
    so that (with distinct scores) exactly m pooled candidates score at or above it.  Returns
    +inf when m = 0."""
    pooled = np.sort(np.concatenate([np.ravel(np.asarray(t, dtype=np.float64))
                                     for t in score_sets]))[::-1]
    m = int(np.floor(frac * pooled.size + 0.5))
    return float(pooled[m - 1]) if m > 0 else float("inf")


def _row(t, j):
    """Row j of a stored [I, H] tensor, keeping its storage form."""
    if isinstance(t, tuple):
        if t[0] == "bf16":
            return ("bf16", t[1][j:j + 1])
        return ("mxfp4", t[1][j:j + 1], t[2][j:j + 1])
    return np.asarray(t)[j:j + 1]


# ----------------------------------------------------------------------------------------
# Batches: the touched-expert union and per-expert token buckets
# ----------------------------------------------------------------------------------------

def union_experts(ids: np.ndarray, E: int):
    """Distinct experts touched by a batch and each expert's (token, slot) list.

    A batch reads every expert that any of its tokens picked [Sparse-501B, section 2].
    Returns n_touched, touched (ascending, length n_touched), offsets [E+1] (prefix sum of
    per-expert counts), slots [B*k] (flat b*k+i, grouped by expert, ascending within one).
    """
    ids = np.asarray(ids, dtype=np.int64)
    B, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    slots = np.empty(B * k, dtype=np.int64)
    fill = offsets[:-1].copy()
    for f in range(B * k):          # ascending flat index -> ascending within each expert
        e = flat[f]
        slots[fill[e]] = f
        fill[e] += 1
    touched = np.nonzero(counts)[0]
    return int(touched.shape[0]), touched, offsets, slots


def expected_touched(E: int, k: int, B: int) -> float:
    """E * [1 - (1 - k/E)^B], experts touched by B tokens each picking k uniformly
    [Sparse-501B, section 2]."""
    return E * (1.0 - (1.0 - k / E) ** B)


def expected_touched_exact(E: int, k: int, B: int) -> Fraction:
    """Mean distinct-expert count over every routing of B tokens (each a k-subset of E),
    by enumeration; exact rational.  Tiny E, k, B only."""
    subsets = list(combinations(range(E), k))
    total = Fraction(0)
    for choice in product(subsets, repeat=B):
        total += len(set().union(*choice))
    return total / (len(subsets) ** B)


def half_touched_batch(E: int, k: int) -> float:
    """Batch at which half the experts are touched, ln2 / (k/E) [Sparse-501B, section 3[B]]."""
    return math.log(2.0) / (k / E)


# ----------------------------------------------------------------------------------------
# Linear experts (one matrix each): the batch-sweep workload
# ----------------------------------------------------------------------------------------

def linear_moe(X: np.ndarray, ids: np.ndarray, w: np.ndarray, get_matrix) -> np.ndarray:
    """Y[b] = sum_i w[b,i] * M_{ids[b,i]} X[b] ("one matmul per expert" [Sparse-501B, 3])."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    cache = {}
    rows = []
    for b in range(X.shape[0]):
        y = 0.0
        for e, we in zip(ids[b], w[b]):
            e = int(e)
            if e not in cache:
                cache[e] = to_f64(get_matrix(e))
            y = y + we * (cache[e] @ X[b])
        rows.append(y)
    return np.stack(rows)


# ----------------------------------------------------------------------------------------
# Byte accounting and the bandwidth ceiling
# ----------------------------------------------------------------------------------------

BYTES_PER_ELEM = {"f32": 4.0, "bf16": 2.0, "mxfp4": 0.5 + 1.0 / 32.0}


def layer_bytes(H, I, k, expert_dtype, n_shared=0, I_shared=0, shared_dtype="bf16",
                E=0, router_dtype=None, n_experts_read=None):
    """Weight bytes one token reads in one layer.

    Only the routed experts' tensors are read (active, not total, parameters), plus the
    shared experts and the router that every token touches [MoE-arith, "Two Numbers"].
    A SwiGLU expert holds 3 * H * I weights.  For a batch, pass the touched count.
    """
    n = k if n_experts_read is None else n_experts_read
    b = n * 3 * H * I * BYTES_PER_ELEM[expert_dtype]
    b += n_shared * 3 * H * I_shared * BYTES_PER_ELEM[shared_dtype or "bf16"]
    if router_dtype is not None:
        b += E * H * BYTES_PER_ELEM[router_dtype]
    return b


def sparse_layer_bytes(H, I, k, keep, expert_dtype, n_shared=0, I_shared=0,
                       shared_dtype="bf16", E=0, router_dtype=None):
    """Bytes of the channel-sparse variant: every gate row (to score), the kept up rows and
    down columns only, the down-norm table entries of the candidates, shared, router."""
    be = BYTES_PER_ELEM[expert_dtype]
    b = k * I * H * be + 2 * keep * H * be + 4 * k * I
    b += n_shared * 3 * H * I_shared * BYTES_PER_ELEM[shared_dtype or "bf16"]
    if router_dtype is not None:
        b += E * H * BYTES_PER_ELEM[router_dtype]
    return b


def decode_ceiling(bandwidth: float, bytes_per_token: float) -> float:
    """Tokens per second when a token costs its bytes at the given bandwidth
    [MoE-arith, "What the Runtime Does With the Promise" and "Code"]."""
    return bandwidth / bytes_per_token


def billed_bytes(offsets, nbytes, sector=32):
    """Bytes billed when every touched sector is fetched whole [Reader, Fig. 2(c)]."""
    touched = set()
    for off, n in zip(offsets, nbytes):
        for s in range(off // sector, (off + n - 1) // sector + 1):
            touched.add(s)
    return len(touched) * sector
