"""Build step for the CPU oracle (test infrastructure only).

Compiles ``zero_oracle.c`` with gcc into ``liboracle.so`` beside it, with the
flags that keep one IEEE rounding per source statement: no contraction of
multiply-add pairs, no fast-math reassociation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zero_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
          "-fno-builtin-rint", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force=True):
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
