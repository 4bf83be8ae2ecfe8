"""Build libdllm.so in place with hipcc for gfx950 (always recompiles)."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdllm.so")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
# Packed-fp32 instructions are turned off for all device code.
# Logits are finite by contract, so NaN handling is compiled out (-fno-honor-nans): max chains
# map to v_max3_f32 without canonicalising each load.  Infinities are still honoured.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17", "-Wall", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def build(verbose=False, extra=()):
    cmd = ["hipcc", *FLAGS, *extra, "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
