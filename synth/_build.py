"""Build step for the GPU half of the synthetic-input generator (libsynth.so)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth_fill.hip")
LIB = os.path.join(HERE, "libsynth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force=True):
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, *FLAGS, SRC, "-o", tmp], check=True,
                   stderr=subprocess.PIPE if not os.environ.get("ZERO_BUILD_VERBOSE") else None)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
