"""Build libzero.so (the C-ABI library) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzero.so")
SOURCES = [os.path.join(CSRC, "zero_kernels.hip"), os.path.join(CSRC, "zero_api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: one rounding per fp32 operation (no fused multiply-add).
# -packed-fp32-ops off: no v_pk_* fp32 instructions are generated.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
         "-fPIC", "-shared", "-fvisibility=hidden", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def build(force=True):
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libzero.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
