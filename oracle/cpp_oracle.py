"""Binding of the plain C++17 oracle (oracle/cpp/moe_oracle.cpp).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may load it.  The functions take and return the same values as their namesakes
in ``oracle.moe_oracle`` (stored tensors as float32/float64 arrays, ("bf16", u16) or
("mxfp4", codes, scales)); all arithmetic happens in the C++ library, in double precision, in
index order.  ``set_threads(n)`` splits independent outputs over n host threads (results do
not depend on n).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "cpp", "moe_oracle.cpp")
LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None
_threads = 1

OC_F64, OC_F32, OC_BF16, OC_MXFP4 = 0, 1, 2, 3


def build(verbose: bool = False) -> str:
    """Compile the oracle for the host (g++, no GPU code)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", SRC,
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class _Tensor(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        vp, lg, i32 = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
        tp = ctypes.POINTER(_Tensor)
        sig = {
            "oc_widen": [tp, lg, lg, vp],
            "oc_router_logits": [vp, lg, lg, tp, lg, i32, vp],
            "oc_route": [vp, lg, lg, lg, vp, vp],
            "oc_expert_activations": [vp, lg, lg, tp, tp, i32, vp],
            "oc_layer_given": [vp, lg, lg, lg, vp, tp, tp, tp, lg, lg, tp, tp, tp, i32, vp],
            "oc_down_norms": [tp, lg, lg, vp],
            "oc_channel_select": [vp, lg, lg, lg, vp, vp, tp, tp, tp, vp, lg, i32, lg, lg, tp,
                                  tp, tp, i32, vp, vp],
            "oc_union_experts": [vp, lg, lg, lg, vp, vp, vp, vp],
            "oc_linear_moe": [vp, lg, lg, lg, lg, vp, vp, tp, lg, i32, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    global _threads
    _threads = max(1, int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class _Stored:
    """A stored tensor as the C struct, with the arrays it points into kept alive."""

    def __init__(self, t):
        if isinstance(t, tuple):
            if t[0] == "bf16":
                d = np.ascontiguousarray(t[1], dtype=np.uint16)
                self.keep = (d,)
                self.shape = d.shape
                self.c = _Tensor(OC_BF16, d.ctypes.data, None)
            elif t[0] == "mxfp4":
                d = np.ascontiguousarray(t[1], dtype=np.uint8)
                s = np.ascontiguousarray(t[2], dtype=np.uint8)
                self.keep = (d, s)
                self.shape = (d.shape[0], d.shape[1] * 2)
                self.c = _Tensor(OC_MXFP4, d.ctypes.data, s.ctypes.data)
            else:
                raise ValueError(t[0])
        else:
            a = np.asarray(t)
            if a.dtype == np.float32:
                d = np.ascontiguousarray(a)
                self.c = _Tensor(OC_F32, d.ctypes.data, None)
            else:
                d = np.ascontiguousarray(a, dtype=np.float64)
                self.c = _Tensor(OC_F64, d.ctypes.data, None)
            self.keep = (d,)
            self.shape = d.shape


def _array_of(stored):
    arr = (_Tensor * max(1, len(stored)))()
    for i, s in enumerate(stored):
        arr[i] = s.c
    return arr


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


# ------------------------------------------------------------------------ storage decoding
def bf16_to_f64(u16):
    u = np.ascontiguousarray(np.atleast_2d(np.asarray(u16, dtype=np.uint16)))
    out = np.empty(u.shape, dtype=np.float64)
    s = _Stored(("bf16", u))
    lib().oc_widen(ctypes.byref(s.c), u.shape[0], u.shape[1], _ptr(out))
    return out.reshape(np.shape(u16))


def mxfp4_to_f64(codes, scales):
    s = _Stored(("mxfp4", codes, scales))
    out = np.empty(s.shape, dtype=np.float64)
    lib().oc_widen(ctypes.byref(s.c), s.shape[0], s.shape[1], _ptr(out))
    return out


# ------------------------------------------------------------------------------- routing
def router_logits(x, w_router):
    x = _f64(np.atleast_2d(x))
    s = _Stored(w_router)
    E, H = s.shape
    out = np.empty((x.shape[0], E), dtype=np.float64)
    lib().oc_router_logits(_ptr(x), x.shape[0], H, ctypes.byref(s.c), E, _threads, _ptr(out))
    return out


def route(logits, k: int):
    l = _f64(np.atleast_2d(logits))
    B, E = l.shape
    ids = np.empty((B, k), dtype=np.int64)
    w = np.empty((B, k), dtype=np.float64)
    if lib().oc_route(_ptr(l), B, E, k, _ptr(ids), _ptr(w)) != 0:
        raise ValueError("k out of range")
    return ids, w


def silu(z):
    """Test-side helper (numpy): the gate nonlinearity, for expected values in tests."""
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------- the experts
def expert_activations(x, gate, up):
    x = _f64(np.reshape(x, -1))
    G, V = _Stored(gate), _Stored(up)
    I = G.shape[0]
    a = np.empty(I, dtype=np.float64)
    lib().oc_expert_activations(_ptr(x), x.shape[0], I, ctypes.byref(G.c), ctypes.byref(V.c),
                                _threads, _ptr(a))
    return a


def _layer_given(x, experts, w, shared):
    x = _f64(np.reshape(x, -1))
    H = x.shape[0]
    G = [_Stored(e[0]) for e in experts]
    V = [_Stored(e[1]) for e in experts]
    D = [_Stored(e[2]) for e in experts]
    SG = [_Stored(s[0]) for s in shared]
    SV = [_Stored(s[1]) for s in shared]
    SD = [_Stored(s[2]) for s in shared]
    I = G[0].shape[0] if G else 0
    Is = SG[0].shape[0] if SG else 0
    wv = _f64(np.reshape(np.asarray(w, dtype=np.float64), -1)) if len(experts) else \
        np.zeros(1)
    y = np.empty(H, dtype=np.float64)
    lib().oc_layer_given(_ptr(x), H, I, len(experts), _ptr(wv), _array_of(G), _array_of(V),
                         _array_of(D), len(shared), Is, _array_of(SG), _array_of(SV),
                         _array_of(SD), _threads, _ptr(y))
    return y


def expert_output(x, gate, up, down_t):
    return _layer_given(x, [(gate, up, down_t)], [1.0], [])


def moe_layer_token(x, w_router, get_expert, k, shared=(), logits=None):
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    if logits is None:
        logits = router_logits(x, w_router)[0]
    ids, w = route(np.asarray(logits)[None, :], k)
    ids, w = ids[0], w[0]
    y = _layer_given(x, [get_expert(int(e)) for e in ids], w, list(shared))
    return y, ids, w


def moe_layer_given(x, ids, w, get_expert, shared=()):
    return _layer_given(x, [get_expert(int(e)) for e in ids], w, list(shared))


# -------------------------------------------------------------------- channel selection
def down_norms(down_t):
    D = _Stored(down_t)
    I, H = D.shape
    out = np.empty(I, dtype=np.float64)
    lib().oc_down_norms(ctypes.byref(D.c), I, H, _ptr(out))
    return out


def channel_select_token(x, ids, w, get_expert, dnorm_of, keep, shared=(),
                         mode="gate_dnorm"):
    if mode not in ("gate_dnorm", "router_weighted"):
        raise ValueError(mode)
    x = _f64(np.reshape(x, -1))
    H = x.shape[0]
    ids = np.ascontiguousarray(np.reshape(ids, -1), dtype=np.int64)
    wv = _f64(np.reshape(w, -1))
    k = ids.shape[0]
    ex = [get_expert(int(e)) for e in ids]
    G = [_Stored(e[0]) for e in ex]
    V = [_Stored(e[1]) for e in ex]
    D = [_Stored(e[2]) for e in ex]
    I = G[0].shape[0]
    dn = _f64(np.stack([np.asarray(dnorm_of(int(e)), dtype=np.float64) for e in ids]))
    SG = [_Stored(s[0]) for s in shared]
    SV = [_Stored(s[1]) for s in shared]
    SD = [_Stored(s[2]) for s in shared]
    Is = SG[0].shape[0] if SG else 0
    kept = np.empty(max(keep, 1), dtype=np.int64)
    y = np.empty(H, dtype=np.float64)
    r = lib().oc_channel_select(_ptr(x), H, I, k, _ptr(ids), _ptr(wv), _array_of(G),
                                _array_of(V), _array_of(D), _ptr(dn), keep,
                                1 if mode == "router_weighted" else 0, len(SG), Is,
                                _array_of(SG), _array_of(SV), _array_of(SD), _threads,
                                _ptr(kept), _ptr(y))
    if r != 0:
        raise ValueError("keep out of range")
    return kept[:keep], y


# ------------------------------------------------------------------------------- batches
def union_experts(ids, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    B, k = ids.shape
    n = np.zeros(1, dtype=np.int64)
    touched = np.empty(E, dtype=np.int64)
    offsets = np.empty(E + 1, dtype=np.int64)
    slots = np.empty(B * k, dtype=np.int64)
    if lib().oc_union_experts(_ptr(ids), B, k, E, _ptr(n), _ptr(touched), _ptr(offsets),
                              _ptr(slots)) != 0:
        raise ValueError("id out of range")
    nt = int(n[0])
    return nt, touched[:nt], offsets, slots


def linear_moe(X, ids, w, get_matrix):
    X = _f64(np.atleast_2d(X))
    B, H = X.shape
    ids = np.asarray(ids, dtype=np.int64)
    k = ids.shape[1]
    used = sorted({int(e) for e in ids.reshape(-1)})
    local = np.ascontiguousarray(np.vectorize({e: i for i, e in enumerate(used)}.get)(ids),
                                 dtype=np.int64)
    mats = [get_matrix(e) for e in used]
    if isinstance(mats[0], tuple) and mats[0][0] == "bf16":
        M = _Stored(("bf16", np.concatenate([m[1] for m in mats])))
    elif isinstance(mats[0], tuple):
        M = _Stored(("mxfp4", np.concatenate([m[1] for m in mats]),
                     np.concatenate([m[2] for m in mats])))
    else:
        M = _Stored(np.concatenate([np.asarray(m) for m in mats]))
    I = M.shape[0] // len(used)
    wv = _f64(w)
    Y = np.empty((B, I), dtype=np.float64)
    lib().oc_linear_moe(_ptr(X), B, H, I, k, _ptr(local), _ptr(wv), ctypes.byref(M.c),
                        len(used), _threads, _ptr(Y))
    return Y
