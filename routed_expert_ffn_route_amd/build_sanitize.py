"""Sanitizer build of the host code: libmoe_ffn_san.so.

moe_host.hip (descriptor and argument validation, workspace layout, the C ABI) is compiled
with AddressSanitizer and UndefinedBehaviorSanitizer on its host pass only (device code is
never instrumented) and linked with the kernels' objects of the regular build.  The library
needs the clang ASan runtime preloaded (``ASAN_RUNTIME``); the host-validation tests load it
through ``MOE_FFN_LIBRARY``.  Build the regular library first (build.py).
"""
import glob
import os
import subprocess

from .build import CSRC, HERE, HIPCC_FLAGS

SAN_LIB = os.path.join(HERE, "libmoe_ffn_san.so")
ASAN_RUNTIME = (sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/"
                                 "libclang_rt.asan-x86_64.so")) or [""])[-1]
# each sanitizer flag applies to the host pass only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build_sanitized(verbose: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build_san")
    os.makedirs(build_dir, exist_ok=True)
    objs = [o for o in sorted(glob.glob(os.path.join(HERE, "_build", "*.o")))
            if os.path.basename(o) != "moe_host.o"]
    if len(objs) < 7:
        raise RuntimeError("build the regular library (build.py) before the sanitizer build")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    host = os.path.join(build_dir, "moe_host_san.o")
    cmds = [["hipcc", *flags, *SAN_FLAGS, "-c", os.path.join(CSRC, "moe_host.hip"), "-o", host],
            ["hipcc", "-shared", "-fPIC", "--offload-arch=gfx950", host, *objs, *SAN_FLAGS,
             "-Xarch_host", "-shared-libasan", "-o", SAN_LIB + ".tmp"]]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("sanitizer build failed:\n" + r.stderr)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_sanitized(verbose=True))
