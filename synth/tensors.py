"""Workload tensors, element by element the same on the host and on the device.

Host functions return numpy arrays in storage form: float32 arrays, ("bf16", uint16 bits)
or ("mxfp4", codes, scales).  Device functions fill torch tensors on the GPU with the same
bytes.  Layouts match include/moe_ffn.h: expert tensors stacked [E][I][H], rows along H;
shared experts stacked [n_shared][I_s][H]; the router [E][H]; linear experts [E][I][H].
"""
from __future__ import annotations

import numpy as np

from . import (mxfp4, mxfp4_device, normal_bf16, normal_bf16_device, normal_f32,
               normal_f32_device)
from .workloads import Workload, stream_id, x_sub


def _host(dtype, seed, stream, first, n, sigma, shape):
    if dtype == "f32":
        return normal_f32(seed, stream, first, n, sigma).reshape(shape)
    if dtype == "bf16":
        return ("bf16", normal_bf16(seed, stream, first, n, sigma).reshape(shape))
    raise ValueError(dtype)


def _host_rows(dtype, seed, stream, row0, rows, cols, sigma):
    if dtype == "mxfp4":
        c, s = mxfp4(seed, stream, row0, rows, cols, sigma)
        return ("mxfp4", c, s)
    return _host(dtype, seed, stream, row0 * cols, rows * cols, sigma, (rows, cols))


# ------------------------------------------------------------------------------ host side
def router(wl: Workload, layer: int):
    return _host_rows(wl.router_dtype, wl.seed, stream_id(wl.wwid, "router", layer), 0, wl.E,
                      wl.H, wl.sigma_router)


def expert(wl: Workload, layer: int, e: int):
    """(G_e, V_e, D_e^T), each [I, H] in storage form."""
    out = []
    for kind, sig in (("gate", wl.sigma_gate), ("up", wl.sigma_up), ("down_t", wl.sigma_down)):
        out.append(_host_rows(wl.expert_dtype, wl.seed, stream_id(wl.wwid, kind, layer),
                              e * wl.I, wl.I, wl.H, sig))
    return tuple(out)


def shared(wl: Workload, layer: int, s: int):
    out = []
    for kind, sig in (("sh_gate", wl.sigma_gate), ("sh_up", wl.sigma_up),
                      ("sh_down_t", wl.sigma_down)):
        out.append(_host_rows(wl.shared_dtype, wl.seed, stream_id(wl.wwid, kind, layer),
                              s * wl.I_shared, wl.I_shared, wl.H, sig))
    return tuple(out)


def linear(wl: Workload, e: int):
    return _host_rows(wl.expert_dtype, wl.seed, stream_id(wl.wwid, "linear", 0), e * wl.I,
                      wl.I, wl.H, wl.sigma_gate)


def rotation_signs(wl: Workload, layer: int) -> np.ndarray:
    """The random signs of a layer's block Hadamard rotation: H values in {-1, +1} (int8), the
    sign of the generator's draw (a draw of exactly 0 counts as +1)."""
    v = normal_f32(wl.seed, stream_id(wl.wwid, "signs", layer), 0, wl.H, 1.0)
    return np.where(v < 0, -1, 1).astype(np.int8)


def x(wl: Workload, token: int, layer: int = 0, attempt: int = 0, case: int = 0):
    return normal_f32(wl.seed, stream_id(wl.wid, "x", layer, x_sub(token, attempt, case)), 0,
                      wl.H, wl.sigma_x)


def logits(wl: Workload, token: int, attempt: int = 0, case: int = 0):
    return normal_f32(wl.seed, stream_id(wl.wid, "logits", 0, x_sub(token, attempt, case)), 0,
                      wl.E, wl.sigma_logits)


# ---------------------------------------------------------------------------- device side
def _dev_fill(dtype, seed, stream, first_row, rows, cols, sigma, t, scales=None):
    """Fill tensor t (and scales for MXFP4) with rows [first_row, first_row+rows)."""
    import torch
    hs = torch.cuda.current_stream().cuda_stream
    if dtype == "f32":
        normal_f32_device(seed, stream, first_row * cols, rows * cols, sigma, t.data_ptr(), hs)
    elif dtype == "bf16":
        normal_bf16_device(seed, stream, first_row * cols, rows * cols, sigma, t.data_ptr(), hs)
    elif dtype == "mxfp4":
        mxfp4_device(seed, stream, first_row, rows, cols, sigma, t.data_ptr(),
                     scales.data_ptr(), hs)
    else:
        raise ValueError(dtype)


def _dev_alloc(dtype, rows, cols):
    import torch
    if dtype == "f32":
        return torch.empty((rows, cols), dtype=torch.float32, device="cuda"), None
    if dtype == "bf16":
        return torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"), None
    if dtype == "mxfp4":
        return (torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda"))
    raise ValueError(dtype)


def device_layer(wl: Workload, layer: int) -> dict:
    """All weights of one layer on the device, keyed as the C ABI's moe_weights fields."""
    t = {}
    if wl.router_dtype is not None:
        r, _ = _dev_alloc(wl.router_dtype, wl.E, wl.H)
        _dev_fill(wl.router_dtype, wl.seed, stream_id(wl.wwid, "router", layer), 0, wl.E,
                  wl.H, wl.sigma_router, r)
        t["router"] = r
    if wl.kind == "linear":
        m, _ = _dev_alloc(wl.expert_dtype, wl.E * wl.I, wl.H)
        _dev_fill(wl.expert_dtype, wl.seed, stream_id(wl.wwid, "linear", 0), 0, wl.E * wl.I,
                  wl.H, wl.sigma_gate, m)
        t["linear"] = m
        return t
    for kind, sig in (("gate", wl.sigma_gate), ("up", wl.sigma_up), ("down_t", wl.sigma_down)):
        m, s = _dev_alloc(wl.expert_dtype, wl.E * wl.I, wl.H)
        _dev_fill(wl.expert_dtype, wl.seed, stream_id(wl.wwid, kind, layer), 0, wl.E * wl.I,
                  wl.H, sig, m, s)
        t[kind] = m
        if s is not None:
            t[kind.replace("_t", "") + "_scale"] = s
    if wl.n_shared:
        for kind, sig in (("sh_gate", wl.sigma_gate), ("sh_up", wl.sigma_up),
                          ("sh_down_t", wl.sigma_down)):
            m, _ = _dev_alloc(wl.shared_dtype, wl.n_shared * wl.I_shared, wl.H)
            _dev_fill(wl.shared_dtype, wl.seed, stream_id(wl.wwid, kind, layer), 0,
                      wl.n_shared * wl.I_shared, wl.H, sig, m)
            t[kind] = m
    return t


def device_x(wl: Workload, tokens, layer: int = 0, attempts=None, case: int = 0):
    """[len(tokens), H] float32 device tensor of the tokens' activations."""
    import torch
    out = torch.empty((len(tokens), wl.H), dtype=torch.float32, device="cuda")
    hs = torch.cuda.current_stream().cuda_stream
    for i, tok in enumerate(tokens):
        a = 0 if attempts is None else attempts[i]
        normal_f32_device(wl.seed, stream_id(wl.wid, "x", layer, x_sub(tok, a, case)), 0, wl.H,
                          wl.sigma_x, out[i].data_ptr(), hs)
    return out


def device_logits(wl: Workload, tokens, attempts=None, case: int = 0):
    import torch
    out = torch.empty((len(tokens), wl.E), dtype=torch.float32, device="cuda")
    hs = torch.cuda.current_stream().cuda_stream
    for i, tok in enumerate(tokens):
        a = 0 if attempts is None else attempts[i]
        normal_f32_device(wl.seed, stream_id(wl.wid, "logits", 0, x_sub(tok, a, case)), 0,
                          wl.E, wl.sigma_logits, out[i].data_ptr(), hs)
    return out


def reduced(wl: Workload, **changes) -> Workload:
    """A smaller copy of a workload (same recipe, other sizes) for quick parity cases."""
    import dataclasses
    return dataclasses.replace(wl, **changes)


__all__ = ["router", "expert", "shared", "linear", "x", "logits", "rotation_signs",
           "device_layer", "device_x",
           "device_logits", "reduced", "np"]
