"""Routed-expert FFN layer for MI355X (gfx950): Python binding of the C ABI in include/moe_ffn.h.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_ffn.so``.  Torch tensors supply device memory and streams.  There is no fallback:
if the native library is missing, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ffn.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
DTYPE_NONE, F32, BF16, MXFP4 = -1, 0, 1, 2
SWIGLU, LINEAR = 0, 1
SCORE_GATE_DNORM, SCORE_ROUTER_WEIGHTED = 0, 1

DTYPES = {None: DTYPE_NONE, "f32": F32, "bf16": BF16, "mxfp4": MXFP4}

# Every symbol include/moe_ffn.h declares.
EXPORTS = (
    "moe_layer_workspace_bytes", "moe_layer_create", "moe_layer_destroy", "moe_route",
    "moe_ffn_forward", "moe_channel_select", "moe_union_experts", "moe_layer_check",
    "moe_layer_geometry", "moe_status_string", "moe_last_error",
)


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_experts", "top_k", "inter", "n_shared", "shared_inter", "kind",
        "router_dtype", "expert_dtype", "shared_dtype", "max_batch")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router", "gate", "up", "down_t", "gate_scale", "up_scale", "down_scale", "linear",
        "sh_gate", "sh_up", "sh_down_t")]


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libmoe_ffn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python routed_expert_ffn_route_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_layer_create.restype = i32
        L.moe_layer_create.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(Weights), vp,
                                       sz, vp, ctypes.POINTER(vp)]
        L.moe_layer_destroy.restype = i32
        L.moe_layer_destroy.argtypes = [vp]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp]
        L.moe_ffn_forward.restype = i32
        L.moe_ffn_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.moe_channel_select.restype = i32
        L.moe_channel_select.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
        L.moe_union_experts.restype = i32
        L.moe_union_experts.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_layer_check.restype = i32
        L.moe_layer_check.argtypes = [vp, vp, ctypes.POINTER(i32)]
        L.moe_layer_geometry.restype = i32
        L.moe_layer_geometry.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_desc(H, E, k, I, n_shared=0, I_shared=0, kind=SWIGLU, router_dtype="bf16",
              expert_dtype="bf16", shared_dtype="bf16", max_batch=1) -> LayerDesc:
    return LayerDesc(H, E, k, I, n_shared, I_shared, kind, DTYPES[router_dtype],
                     DTYPES[expert_dtype], DTYPES[shared_dtype] if n_shared else F32,
                     max_batch)


def workspace_bytes(desc: LayerDesc) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(desc)))


class Layer:
    """A routed-expert FFN layer over caller-owned device tensors.

    ``tensors`` maps weight names (router, gate, up, down_t, gate_scale, up_scale,
    down_scale, linear, sh_gate, sh_up, sh_down_t) to device tensors laid out as in
    include/moe_ffn.h.  The workspace is a uint8 device tensor owned by this object, or the
    caller's ``workspace`` (at least workspace_bytes(desc) + 256 bytes), kept alive here.
    """

    def __init__(self, desc: LayerDesc, tensors: dict, stream=None, workspace=None):
        import torch
        self.desc = desc
        self.tensors = dict(tensors)  # keep the weights alive
        nbytes = workspace_bytes(desc)
        if nbytes == 0:
            raise MoeError(MOE_ERR_ARG, "invalid layer descriptor")
        if workspace is None:
            workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        elif workspace.numel() * workspace.element_size() < nbytes + 256:
            raise MoeError(MOE_ERR_ARG, "workspace too small")
        self.workspace = workspace
        off = (-self.workspace.data_ptr()) % 256
        self._ws_ptr = self.workspace.data_ptr() + off
        self._ws_bytes = nbytes
        w = Weights(*[None if self.tensors.get(n) is None else self.tensors[n].data_ptr()
                      for n, _ in Weights._fields_])
        h = ctypes.c_void_p()
        _check(lib().moe_layer_create(ctypes.byref(desc), ctypes.byref(w),
                                      ctypes.c_void_p(self._ws_ptr), nbytes, _stream(stream),
                                      ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def route(self, x=None, logits_in=None, B=None, ids=None, w=None, logits_out=None,
              stream=None):
        src = x if x is not None else logits_in
        B = src.shape[0] if B is None else B
        _check(lib().moe_route(self.handle, _ptr(x), _ptr(logits_in), B, _ptr(ids), _ptr(w),
                               _ptr(logits_out), _stream(stream)))

    def forward(self, x, y, ids=None, w=None, B=None, stream=None):
        B = x.shape[0] if B is None else B
        _check(lib().moe_ffn_forward(self.handle, _ptr(x), B, _ptr(ids), _ptr(w), _ptr(y),
                                     _stream(stream)))

    def channel_select(self, x, keep, kept, y=None, ids=None, w=None,
                       mode=SCORE_GATE_DNORM, stream=None):
        _check(lib().moe_channel_select(self.handle, _ptr(x), _ptr(ids), _ptr(w), keep, mode,
                                        _ptr(kept), _ptr(y), _stream(stream)))

    def check(self, stream=None) -> int:
        err = ctypes.c_int32(0)
        _check(lib().moe_layer_check(self.handle, _stream(stream), ctypes.byref(err)))
        return err.value

    def geometry(self):
        wg, th = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().moe_layer_geometry(self.handle, ctypes.byref(wg), ctypes.byref(th)))
        return wg.value, th.value


def union_experts(ids, E, n_touched, touched, offsets, slots, stream=None):
    B, k = ids.shape
    _check(lib().moe_union_experts(_ptr(ids), B, k, E, _ptr(n_touched), _ptr(touched),
                                   _ptr(offsets), _ptr(slots), _stream(stream)))
