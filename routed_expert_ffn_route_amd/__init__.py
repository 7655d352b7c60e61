"""Routed-expert FFN layer for MI355X (gfx950): Python binding of the C ABI in include/moe_ffn.h.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_ffn.so``.  Torch tensors supply device memory and streams.  There is no fallback:
if the native library is missing, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_FFN_LIBRARY names another build of the same library (the sanitizer build of the host
# code, libmoe_ffn_san.so, is loaded this way by the host-validation tests)
LIB_PATH = os.environ.get("MOE_FFN_LIBRARY") or os.path.join(_HERE, "libmoe_ffn.so")
SAN_LIB_PATH = os.path.join(_HERE, "libmoe_ffn_san.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
DTYPE_NONE, F32, BF16, MXFP4 = -1, 0, 1, 2
SWIGLU, LINEAR = 0, 1
SCORE_GATE_DNORM, SCORE_ROUTER_WEIGHTED = 0, 1

DTYPES = {None: DTYPE_NONE, "f32": F32, "bf16": BF16, "mxfp4": MXFP4}

# Every symbol include/moe_ffn.h declares.
EXPORTS = (
    "moe_layer_workspace_bytes", "moe_layer_create", "moe_layer_destroy", "moe_route",
    "moe_ffn_forward", "moe_ffn_forward_noalloc", "moe_channel_select", "moe_union_experts",
    "moe_layer_routing", "moe_sketch_bytes", "moe_layer_build_sketch",
    "moe_channel_select_sketch", "moe_channel_select_threshold", "moe_layer_scores",
    "moe_recovery_bytes", "moe_layer_build_recovery", "moe_channel_select_reader",
    "moe_channel_select_batch", "moe_layer_check", "moe_layer_geometry", "moe_status_string", "moe_last_error",
)
# The phase-timeline build (libmoe_ffn_timeline.so) exports one more, for measurement only.
TIMELINE_LIB_PATH = os.path.join(_HERE, "libmoe_ffn_timeline.so")


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


def use_timeline_library():
    """Load the phase-timeline build instead of libmoe_ffn.so (before any other call):
    the same kernels with per-workgroup phase stamps compiled in (bench.py --timeline)."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("a library is already loaded")
    LIB_PATH = TIMELINE_LIB_PATH
    L = lib()
    L.moe_debug_set_stamps.restype = ctypes.c_int32
    L.moe_debug_set_stamps.argtypes = [ctypes.c_void_p]
    return L


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
        L.moe_ffn_forward_noalloc.restype = i32
        L.moe_ffn_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(Weights),
                                              vp, i32, vp, vp, vp, vp]
        L.moe_channel_select.restype = i32
        L.moe_channel_select.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
        L.moe_union_experts.restype = i32
        L.moe_union_experts.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_layer_routing.restype = i32
        L.moe_layer_routing.argtypes = [vp, i32, vp, vp, vp]
        L.moe_sketch_bytes.restype = sz
        L.moe_sketch_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_layer_build_sketch.restype = i32
        L.moe_layer_build_sketch.argtypes = [vp, vp, vp, sz, vp]
        L.moe_channel_select_sketch.restype = i32
        L.moe_channel_select_sketch.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
        L.moe_channel_select_threshold.restype = i32
        L.moe_channel_select_threshold.argtypes = [vp, vp, vp, vp, ctypes.c_float, i32, vp, vp,
                                                   vp, vp]
        L.moe_layer_scores.restype = i32
        L.moe_layer_scores.argtypes = [vp, vp, vp]
        L.moe_recovery_bytes.restype = sz
        L.moe_recovery_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_layer_build_recovery.restype = i32
        L.moe_layer_build_recovery.argtypes = [vp, vp, i32, vp, sz, vp]
        L.moe_channel_select_reader.restype = i32
        L.moe_channel_select_reader.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
        L.moe_channel_select_batch.restype = i32
        L.moe_channel_select_batch.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, vp, vp]
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


def _need(t, name, dtype, shape=None, min_numel=None):
    """Reject a tensor the kernels would misread or overrun: it must be a contiguous CUDA
    tensor of `dtype`, with `shape` (None entries match any size) or at least `min_numel`
    elements.  Raises MoeError(MOE_ERR_ARG) before any native call."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise MoeError(MOE_ERR_ARG, f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise MoeError(MOE_ERR_ARG, f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise MoeError(MOE_ERR_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(MOE_ERR_ARG, f"{name} must be contiguous")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            raise MoeError(MOE_ERR_ARG, f"{name} has shape {tuple(t.shape)}, needs {shape}")
    if min_numel is not None and t.numel() < min_numel:
        raise MoeError(MOE_ERR_ARG, f"{name} has {t.numel()} elements, needs {min_numel}")


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
        import torch
        d = self.desc
        src = x if x is not None else logits_in
        if src is None:
            raise MoeError(MOE_ERR_ARG, "one of x and logits_in must be given")
        B = src.shape[0] if B is None else B
        if x is not None:
            _need(x, "x", torch.float32, min_numel=B * d.hidden)
        if logits_in is not None:
            _need(logits_in, "logits_in", torch.float32, min_numel=B * d.n_experts)
        _need(ids, "ids", torch.int32, min_numel=B * d.top_k)
        _need(w, "w", torch.float32, min_numel=B * d.top_k)
        if logits_out is not None:
            _need(logits_out, "logits_out", torch.float32, min_numel=B * d.n_experts)
        _check(lib().moe_route(self.handle, _ptr(x), _ptr(logits_in), B, _ptr(ids), _ptr(w),
                               _ptr(logits_out), _stream(stream)))

    def forward(self, x, y, ids=None, w=None, B=None, stream=None):
        import torch
        d = self.desc
        B = x.shape[0] if B is None else B
        out_dim = d.inter if d.kind == LINEAR else d.hidden
        _need(x, "x", torch.float32, min_numel=B * d.hidden)
        _need(y, "y", torch.float32, min_numel=B * out_dim)
        if ids is not None:
            _need(ids, "ids", torch.int32, min_numel=B * d.top_k)
        if w is not None:
            _need(w, "w", torch.float32, min_numel=B * d.top_k)
        _check(lib().moe_ffn_forward(self.handle, _ptr(x), B, _ptr(ids), _ptr(w), _ptr(y),
                                     _stream(stream)))

    def build_sketch(self, signs, stream=None):
        """moe_layer_build_sketch: allocate the sketch buffer (torch) and build it from the
        rotation signs (int8 [H] on the device); both are kept alive by the handle."""
        import torch
        d = self.desc
        _need(signs, "signs", torch.int8, min_numel=d.hidden)
        n = lib().moe_sketch_bytes(ctypes.byref(d))
        if n == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED, "this layer has no sketch form")
        buf = torch.empty(n + 256, dtype=torch.uint8, device=signs.device)
        off = (-buf.data_ptr()) % 256
        self._sketch = (buf, signs, off)
        _check(lib().moe_layer_build_sketch(self.handle, _ptr(signs),
                                            ctypes.c_void_p(buf.data_ptr() + off), n,
                                            _stream(stream)))
        return buf[off:off + n]

    def build_recovery(self, U, stream=None):
        """moe_layer_build_recovery: allocate the recovery buffer (torch) and build it from U
        (float32 [H][32] on the device); both are kept alive by the handle."""
        import torch
        d = self.desc
        _need(U, "U", torch.float32, min_numel=d.hidden * 32)
        n = lib().moe_recovery_bytes(ctypes.byref(d))
        if n == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED, "this layer has no recovery form")
        buf = torch.empty(n + 256, dtype=torch.uint8, device=U.device)
        off = (-buf.data_ptr()) % 256
        self._recovery = (buf, U)
        _check(lib().moe_layer_build_recovery(self.handle, _ptr(U), 32,
                                              ctypes.c_void_p(buf.data_ptr() + off), n,
                                              _stream(stream)))
        return buf[off:off + n]

    def channel_select(self, x, keep, kept, y=None, ids=None, w=None,
                       mode=SCORE_GATE_DNORM, stream=None, sketch=False, reader=False):
        """moe_channel_select, with sketch=True moe_channel_select_sketch, with reader=True
        moe_channel_select_reader (sketch screen plus recovery)."""
        import torch
        d = self.desc
        _need(x, "x", torch.float32, min_numel=d.hidden)
        if kept is not None or keep > 0:
            _need(kept, "kept", torch.int32, min_numel=keep)
        if y is not None:
            _need(y, "y", torch.float32, min_numel=d.hidden)
        if ids is not None:
            _need(ids, "ids", torch.int32, min_numel=d.top_k)
        if w is not None:
            _need(w, "w", torch.float32, min_numel=d.top_k)
        fn = (lib().moe_channel_select_reader if reader else
              lib().moe_channel_select_sketch if sketch else lib().moe_channel_select)
        _check(fn(self.handle, _ptr(x), _ptr(ids), _ptr(w), keep, mode, _ptr(kept), _ptr(y),
                  _stream(stream)))

    def channel_select_threshold(self, x, tau, kept, kept_count, y=None, ids=None, w=None,
                                 mode=SCORE_GATE_DNORM, stream=None):
        """moe_channel_select_threshold: keep every candidate scoring at least tau."""
        import torch
        d = self.desc
        _need(x, "x", torch.float32, min_numel=d.hidden)
        _need(kept, "kept", torch.int32, min_numel=d.top_k * d.inter)
        _need(kept_count, "kept_count", torch.int32, min_numel=1)
        if y is not None:
            _need(y, "y", torch.float32, min_numel=d.hidden)
        if ids is not None:
            _need(ids, "ids", torch.int32, min_numel=d.top_k)
        if w is not None:
            _need(w, "w", torch.float32, min_numel=d.top_k)
        _check(lib().moe_channel_select_threshold(self.handle, _ptr(x), _ptr(ids), _ptr(w),
                                                  float(tau), mode, _ptr(kept),
                                                  _ptr(kept_count), _ptr(y), _stream(stream)))

    def channel_select_batch(self, x, keep, kept, y, kept_count=None, ids=None, w=None,
                             stream=None):
        """moe_channel_select_batch: one kept channel set for the batch x [B][H]."""
        import torch
        d = self.desc
        B = x.shape[0]
        _need(x, "x", torch.float32, min_numel=B * d.hidden)
        _need(y, "y", torch.float32, min_numel=B * d.hidden)
        if kept is not None or keep > 0:
            _need(kept, "kept", torch.int32, min_numel=keep)
        if kept_count is not None:
            _need(kept_count, "kept_count", torch.int32, min_numel=1)
        if ids is not None:
            _need(ids, "ids", torch.int32, min_numel=B * d.top_k)
        if w is not None:
            _need(w, "w", torch.float32, min_numel=B * d.top_k)
        _check(lib().moe_channel_select_batch(self.handle, _ptr(x), B, _ptr(ids), _ptr(w), keep,
                                              _ptr(kept), _ptr(kept_count), _ptr(y),
                                              _stream(stream)))

    def scores(self, out, stream=None):
        """moe_layer_scores: the last channel-selection call's k*I scores, slot-major."""
        import torch
        _need(out, "scores", torch.float32, min_numel=self.desc.top_k * self.desc.inter)
        _check(lib().moe_layer_scores(self.handle, _ptr(out), _stream(stream)))

    def routing(self, ids, w, B=1, stream=None):
        """Copy the routing the last call used into ids, w [B][k] (moe_layer_routing)."""
        import torch
        _need(ids, "ids", torch.int32, min_numel=B * self.desc.top_k)
        _need(w, "w", torch.float32, min_numel=B * self.desc.top_k)
        _check(lib().moe_layer_routing(self.handle, B, _ptr(ids), _ptr(w), _stream(stream)))

    def check(self, stream=None) -> int:
        err = ctypes.c_int32(0)
        _check(lib().moe_layer_check(self.handle, _stream(stream), ctypes.byref(err)))
        return err.value

    def geometry(self):
        wg, th = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().moe_layer_geometry(self.handle, ctypes.byref(wg), ctypes.byref(th)))
        return wg.value, th.value


def forward_noalloc(desc: LayerDesc, tensors: dict, x, y, ids=None, w=None, B=None,
                    stream=None):
    """moe_ffn_forward_noalloc: the layer without a handle or workspace (the library's static
    scratch); `tensors` as for Layer."""
    import torch
    B = x.shape[0] if B is None else B
    out_dim = desc.inter if desc.kind == LINEAR else desc.hidden
    _need(x, "x", torch.float32, min_numel=B * desc.hidden)
    _need(y, "y", torch.float32, min_numel=B * out_dim)
    if ids is not None:
        _need(ids, "ids", torch.int32, min_numel=B * desc.top_k)
    if w is not None:
        _need(w, "w", torch.float32, min_numel=B * desc.top_k)
    wts = Weights(*[None if tensors.get(n) is None else tensors[n].data_ptr()
                    for n, _ in Weights._fields_])
    _check(lib().moe_ffn_forward_noalloc(ctypes.byref(desc), ctypes.byref(wts), _ptr(x), B,
                                         _ptr(ids), _ptr(w), _ptr(y), _stream(stream)))


def union_experts(ids, E, n_touched, touched, offsets, slots, stream=None):
    import torch
    _need(ids, "ids", torch.int32, shape=(None, None))
    B, k = ids.shape
    _need(n_touched, "n_touched", torch.int32, min_numel=1)
    _need(touched, "touched", torch.int32, min_numel=E)
    _need(offsets, "offsets", torch.int32, min_numel=E + 1)
    _need(slots, "slots", torch.int32, min_numel=B * k)
    _check(lib().moe_union_experts(_ptr(ids), B, k, E, _ptr(n_touched), _ptr(touched),
                                   _ptr(offsets), _ptr(slots), _stream(stream)))
