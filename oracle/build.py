"""Build the CPU oracles (plain C, gcc): oracle/librope_oracle.so (QK rotary
embedding) and oracle/libglu_oracle.so (SwiGLU / GeGLU).

Test infrastructure: building the checker is not using it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rope_oracle.c")
LIB_PATH = os.path.join(HERE, "librope_oracle.so")
GLU_SRC = os.path.join(HERE, "glu_oracle.c")
GLU_LIB_PATH = os.path.join(HERE, "libglu_oracle.so")

# -ffp-contract=off: every product and sum is rounded as written (no FMA).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall"]


def build(src: str = SRC, out: str = LIB_PATH) -> str:
    """Compile ``src`` (default: the oracle) to the shared library ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build_all() -> None:
    build(SRC, LIB_PATH)
    build(GLU_SRC, GLU_LIB_PATH)


if __name__ == "__main__":
    build_all()
    print(LIB_PATH)
    print(GLU_LIB_PATH)
