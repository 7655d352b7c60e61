"""Compile the seeded input generator (synth.hip) into synth/libsynth.so for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "synth.hip")
    cmd = ["hipcc", *HIPCC_FLAGS, src, "-o", LIB + ".tmp", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for synth.hip:\n" + "\n".join(noise))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
