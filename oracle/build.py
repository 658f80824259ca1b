"""Build the CPU oracle (plain C, gcc) into oracle/librope_oracle.so.

Test infrastructure: building the checker is not using it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rope_oracle.c")
LIB_PATH = os.path.join(HERE, "librope_oracle.so")

# -ffp-contract=off: every product and sum is rounded as written (no FMA).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall"]


def build(src: str = SRC, out: str = LIB_PATH) -> str:
    """Compile ``src`` (default: the oracle) to the shared library ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
