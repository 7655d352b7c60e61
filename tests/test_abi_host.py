"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the
host before any HIP call (CPU only: no call here reaches the device)."""
import ctypes
import os
import re

import pytest

import routed_expert_ffn_route_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_ffn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(M.EXPORTS) == names


def test_status_strings():
    lib = M.lib()
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def _desc(**kw):
    base = dict(H=2048, E=256, k=8, I=768, n_shared=1, I_shared=768)
    base.update(kw)
    return M.make_desc(**base)


def test_workspace_bytes_arithmetic():
    d = _desc()
    n = M.workspace_bytes(d)
    assert n > 0 and n % 256 == 0
    # dnorm [E][I] fp32 and the partial rows (512 x H fp32) dominate
    assert n >= 256 * 768 * 4 + 512 * 2048 * 4
    assert M.workspace_bytes(_desc(H=4096)) > n
    bigger = _desc()
    bigger.max_batch = 64
    assert M.workspace_bytes(bigger) > n
    for bad in (dict(H=100), dict(E=0), dict(k=0), dict(k=300), dict(I=7), dict(k=40),
                dict(n_shared=5)):
        assert M.workspace_bytes(_desc(**bad)) == 0, bad


def test_create_rejects_bad_arguments_without_device():
    lib = M.lib()
    h = ctypes.c_void_p()
    d = _desc()
    w = M.Weights()
    # invalid descriptor
    st = lib.moe_layer_create(ctypes.byref(_desc(H=30)), ctypes.byref(w), None, 0, None,
                              ctypes.byref(h))
    assert st == M.MOE_ERR_ARG
    assert b"hidden" in lib.moe_last_error()
    # missing weights
    st = lib.moe_layer_create(ctypes.byref(d), ctypes.byref(w), None, 0, None, ctypes.byref(h))
    assert st == M.MOE_ERR_ARG
    # misaligned weights
    w2 = M.Weights(router=0x1000, gate=0x2008, up=0x3000, down_t=0x4000, sh_gate=0x5000,
                   sh_up=0x6000, sh_down_t=0x7000)
    st = lib.moe_layer_create(ctypes.byref(d), ctypes.byref(w2), 0x10000, 1 << 30, None,
                              ctypes.byref(h))
    assert st == M.MOE_ERR_ARG
    # workspace problems
    w3 = M.Weights(router=0x1000, gate=0x2000, up=0x3000, down_t=0x4000, sh_gate=0x5000,
                   sh_up=0x6000, sh_down_t=0x7000)
    st = lib.moe_layer_create(ctypes.byref(d), ctypes.byref(w3), 0x10010, 1 << 30, None,
                              ctypes.byref(h))
    assert st == M.MOE_ERR_WORKSPACE
    st = lib.moe_layer_create(ctypes.byref(d), ctypes.byref(w3), 0x10000, 1024, None,
                              ctypes.byref(h))
    assert st == M.MOE_ERR_WORKSPACE
    # MXFP4 without scales
    dm = _desc()
    dm.expert_dtype = M.MXFP4
    st = lib.moe_layer_create(ctypes.byref(dm), ctypes.byref(w3), 0x10000, 1 << 30, None,
                              ctypes.byref(h))
    assert st == M.MOE_ERR_ARG
    assert not h.value


def test_calls_reject_null_or_destroyed_handles():
    lib = M.lib()
    assert lib.moe_route(None, None, None, 1, None, None, None, None) == M.MOE_ERR_ARG
    assert lib.moe_ffn_forward(None, None, 1, None, None, None, None) == M.MOE_ERR_ARG
    assert lib.moe_channel_select(None, None, None, None, 1, 0, None, None, None) == M.MOE_ERR_ARG
    assert lib.moe_layer_destroy(None) == M.MOE_ERR_ARG
    err = ctypes.c_int32()
    assert lib.moe_layer_check(None, None, ctypes.byref(err)) == M.MOE_ERR_ARG


def test_union_rejects_bad_sizes():
    lib = M.lib()
    p = 0x1000
    assert lib.moe_union_experts(None, 4, 2, 8, p, p, p, p, None) == M.MOE_ERR_ARG
    assert lib.moe_union_experts(p, 0, 2, 8, p, p, p, p, None) == M.MOE_ERR_ARG
    assert lib.moe_union_experts(p, 4, 9, 8, p, p, p, p, None) == M.MOE_ERR_ARG
    assert lib.moe_union_experts(p, 4096, 2, 4096, p, p, p, p, None) == M.MOE_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(M, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        M.lib()


def test_host_validation_under_asan_ubsan():
    """The tests above, run again in a child process against libmoe_ffn_san.so: the host
    code built with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts the
    child with a nonzero status).  The child also confirms that it mapped that library and
    the ASan runtime."""
    import subprocess
    import sys
    from routed_expert_ffn_route_amd import build_sanitize as BS
    if not BS.ASAN_RUNTIME:
        pytest.skip("no clang ASan runtime in this image")
    if not os.path.exists(BS.SAN_LIB):
        BS.build_sanitized()
    env = dict(os.environ, MOE_FFN_LIBRARY=BS.SAN_LIB, LD_PRELOAD=BS.ASAN_RUNTIME,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q",
                        "-p", "no:cacheprovider", "-k", "not asan_ubsan"],
                       cwd=root, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "7 passed" in r.stdout, r.stdout[-2000:]
    probe = ("import routed_expert_ffn_route_amd as M; M.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libmoe_ffn_san.so' in m and 'libclang_rt.asan' in m; print('mapped')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "mapped" in r.stdout, r.stderr[-2000:]
