"""Seeded synthetic inputs for the routed-expert FFN layer (test and benchmark infrastructure).

The pages measure trained checkpoints on public benchmarks; none of that is available, so
every weight, activation and logit used by the tests and the benchmark is drawn here from
a counter-based generator (Philox4x32-10, see ``synth.h``).  The same element comes out of
the host functions (used for the oracle) and the device functions (used to fill GPU memory)
bit for bit.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, stream_id, KIND  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run synth/build.py")
        L = ctypes.CDLL(_LIB_PATH)
        u64, f32, vp, i32 = ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
        L.synth_scale_for_sigma.restype = f32
        L.synth_scale_for_sigma.argtypes = [ctypes.c_double]
        L.synth_philox4x32_10.restype = None
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        for name in ("synth_normal_f32_host", "synth_normal_bf16_host"):
            getattr(L, name).restype = i32
            getattr(L, name).argtypes = [u64, u64, u64, u64, f32, vp, i32]
        L.synth_mxfp4_host.restype = i32
        L.synth_mxfp4_host.argtypes = [u64, u64, u64, u64, u64, f32, vp, vp, i32]
        for name in ("synth_normal_f32_device", "synth_normal_bf16_device"):
            getattr(L, name).restype = i32
            getattr(L, name).argtypes = [u64, u64, u64, u64, f32, vp, vp]
        L.synth_mxfp4_device.restype = i32
        L.synth_mxfp4_device.argtypes = [u64, u64, u64, u64, u64, f32, vp, vp, vp]
        _lib = L
    return _lib


def scale_for_sigma(sigma: float) -> float:
    return float(lib().synth_scale_for_sigma(float(sigma)))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with {rc}")


def normal_f32(seed, stream, first, n, sigma, nthreads=0) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    _check(lib().synth_normal_f32_host(seed, stream, first, n, scale_for_sigma(sigma),
                                       out.ctypes.data, nthreads), "synth_normal_f32_host")
    return out


def normal_bf16(seed, stream, first, n, sigma, nthreads=0) -> np.ndarray:
    """bf16 bit patterns (uint16)."""
    out = np.empty(int(n), dtype=np.uint16)
    _check(lib().synth_normal_bf16_host(seed, stream, first, n, scale_for_sigma(sigma),
                                        out.ctypes.data, nthreads), "synth_normal_bf16_host")
    return out


def mxfp4(seed, stream, row0, rows, cols, sigma, nthreads=0):
    """(codes [rows, cols/2] uint8, scales [rows, cols/32] uint8)."""
    codes = np.empty((int(rows), int(cols) // 2), dtype=np.uint8)
    scales = np.empty((int(rows), int(cols) // 32), dtype=np.uint8)
    _check(lib().synth_mxfp4_host(seed, stream, row0, rows, cols, scale_for_sigma(sigma),
                                  codes.ctypes.data, scales.ctypes.data, nthreads),
           "synth_mxfp4_host")
    return codes, scales


def normal_f32_device(seed, stream, first, n, sigma, ptr, hip_stream=0):
    _check(lib().synth_normal_f32_device(seed, stream, first, n, scale_for_sigma(sigma),
                                         ptr, hip_stream), "synth_normal_f32_device")


def normal_bf16_device(seed, stream, first, n, sigma, ptr, hip_stream=0):
    _check(lib().synth_normal_bf16_device(seed, stream, first, n, scale_for_sigma(sigma),
                                          ptr, hip_stream), "synth_normal_bf16_device")


def mxfp4_device(seed, stream, row0, rows, cols, sigma, codes_ptr, scales_ptr, hip_stream=0):
    _check(lib().synth_mxfp4_device(seed, stream, row0, rows, cols, scale_for_sigma(sigma),
                                    codes_ptr, scales_ptr, hip_stream), "synth_mxfp4_device")


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (storage conversion only)."""
    return (u16.astype(np.uint32) << 16).view(np.float32)
