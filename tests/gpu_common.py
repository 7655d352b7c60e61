"""Shared helpers of the GPU parity tests: margin-checked inputs and oracle references."""
from __future__ import annotations

import numpy as np

import synth
from synth import tensors as T
from oracle import moe_oracle as O

MARGIN = 1e-3       # minimum gap among the k+1 largest router logits
# Channel scores are in output units (|silu(g)| * ||d||), not logit units; their K-th /
# (K+1)-th gap must exceed this fraction of the largest score (fp32 score error is ~1e-6
# of it).
CH_MARGIN_REL = 1e-4
TOL_BF16 = 2e-3     # max |dy| / ||y_ref||_inf for fp32 / bf16 weights, fp32 accumulation
TOL_MXFP4 = 1e-2


def cuda_ok():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pick_attempt(wl, token, layer=0, case=0, host_router=None, k=None):
    """First redraw of x whose oracle router logits have the required top-k margin."""
    Wr = host_router if host_router is not None else T.router(wl, layer)
    k = wl.k if k is None else k
    for a in range(64):
        x = T.x(wl, token, layer, a, case)
        if O.topk_margin(O.router_logits(x, Wr)[0], k) >= MARGIN:
            return a, x
    raise RuntimeError("no margin-satisfying draw in 64 attempts")


class HostLayer:
    """Lazily generated host copies of one layer's weights (for the oracle)."""

    def __init__(self, wl, layer=0):
        self.wl, self.layer = wl, layer
        self.router = T.router(wl, layer) if wl.router_dtype else None
        self._experts = {}
        self.shared = [T.shared(wl, layer, s) for s in range(wl.n_shared)]

    def expert(self, e):
        if e not in self._experts:
            self._experts[e] = T.expert(self.wl, self.layer, e)
        return self._experts[e]


def rel_err(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y_ref)))


def used_choices(ids_row, E):
    """Choices a token's routing row contributes: ids in [0, E), a repeated expert counted
    once at its first choice (the rule every path of the library applies)."""
    out = []
    for i, e in enumerate(ids_row):
        if 0 <= e < E and e not in ids_row[:i]:
            out.append(i)
    return out


def corrupt(ids_np, E):
    """Copy of a routing with a repeated id in token 0, ids past E in token 1 and below 0 in
    token 2 (tokens past those untouched)."""
    bad = ids_np.copy()
    bad[0, 2] = bad[0, 0]
    bad[1, 1] = E + 3
    bad[2, 0] = -1
    return bad
