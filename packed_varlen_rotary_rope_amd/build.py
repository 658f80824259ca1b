"""Build the HIP library librope_qk.so (QK-RoPE and SwiGLU/GeGLU kernels) for
gfx950 with hipcc (in-tree).

Usage: python packed_varlen_rotary_rope_amd/build.py  (run as a script: importing the
package itself needs the library this builds)
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "rope_qk.hip"), os.path.join(PKG, "csrc", "glu.hip")]
LIB_PATH = os.path.join(PKG, "librope_qk.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every product and sum is rounded as written: the Kahan rotation and the
    # double-double sin/cos rely on it
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_fma_f32 and friends) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(extra_flags=(), out: str = LIB_PATH) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-o", tmp, *SRCS]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
