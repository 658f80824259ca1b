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
    # every product and sum is rounded as written: the Kahan rotation and the
    # double-double sin/cos rely on it
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_fma_f32 and friends) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source flags. The RoPE kernels take the kernel arguments a wave needs before
# its first loads as 13 leading dwords; the compiler preloads those into SGPRs at
# wave launch (gfx950 kernel-argument preload; on firmware without it the compiled
# prologue loads them instead), which shortens every launch's start.
SRC_FLAGS = {
    "rope_qk.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=13"],
}


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(extra_flags=(), out: str = LIB_PATH) -> str:
    """Compile each source to an object with its own flags, then link the library."""
    import tempfile
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in SRCS:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *SRC_FLAGS.get(os.path.basename(src), []),
                   *extra_flags, "-c", "-o", obj, src]
            subprocess.run(cmd, check=True)
            objs.append(obj)
        subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
