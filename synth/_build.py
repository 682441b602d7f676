"""Build step for the GPU half of the synthetic-input generator, the
benchmark's HBM calibration probes and CU-masked streams (libsynth.so), and
the host half of the generator (libsynth_cpu.so)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth_fill.hip")
PROBE_SRC = os.path.join(HERE, "probes.hip")
STREAM_SRC = os.path.join(HERE, "streams.hip")
LIB = os.path.join(HERE, "libsynth.so")
CPU_SRC = os.path.join(HERE, "synth_cpu.c")
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_cpu(force=True):
    if not force and os.path.exists(CPU_LIB):
        return CPU_LIB
    tmp = CPU_LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    CPU_SRC, "-o", tmp], check=True)
    os.replace(tmp, CPU_LIB)
    return CPU_LIB


def build(force=True):
    build_cpu(force)
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, *FLAGS, SRC, PROBE_SRC, STREAM_SRC, "-o", tmp], check=True,
                   stderr=subprocess.PIPE if not os.environ.get("ZERO_BUILD_VERBOSE") else None)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
