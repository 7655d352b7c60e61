"""Compile the gfx950 kernels and the C ABI into routed_expert_ffn_route_amd/libmoe_ffn.so.

``build(timeline=True)`` compiles a second library, libmoe_ffn_timeline.so, with the phase
stamps of the single-launch kernels compiled in (MOE_TIMELINE) and the extra export
``moe_debug_set_stamps``; it serves ``bench.py --timeline`` only.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_ffn.so")
LIB_TIMELINE = os.path.join(HERE, "libmoe_ffn_timeline.so")
LIB_PROBE = os.path.join(HERE, "libmoe_probe.so")  # the benchmark's measurement kernels
SOURCES = ["moe_host.hip", "expert_b1.hip", "channel_sparse.hip", "route.hip",
           "batched_swiglu.hip", "linear_mfma.hip", "linear_gemv.hip", "grouped_tn.hip",
           "sketch.hip"]

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def _compile(src: str, build_dir: str, defines, verbose: bool) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *HIPCC_FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag; that warning is harmless
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def build_probe(verbose: bool = False) -> str:
    """libmoe_probe.so: the read-only stream probe and the empty kernel of bench.py."""
    cmd = ["hipcc", *HIPCC_FLAGS, "-shared", os.path.join(CSRC, "probe.hip"),
           "-o", LIB_PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for probe.hip:\n" + r.stderr)
    os.replace(LIB_PROBE + ".tmp", LIB_PROBE)
    return LIB_PROBE


def build(verbose: bool = False, timeline: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build_timeline" if timeline else "_build")
    lib = LIB_TIMELINE if timeline else LIB
    defines = ["-DMOE_TIMELINE"] if timeline else []
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines, verbose), SOURCES))
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, timeline="--timeline" in sys.argv))
    print(build_probe(verbose=True))
