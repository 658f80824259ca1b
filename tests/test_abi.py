"""C-ABI checks that need no GPU: the library loads and exports every function
include/rope_qk.h declares; host-side validation rejects bad arguments before
any HIP call (no kernel is launched by any call here); the host-computed
inverse frequencies; the generated trig constants."""
import ctypes
import os
import re
import subprocess
import sys

import mpmath
import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_rope_amd as rope
from oracle_checks import ref_inv_freq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rope_qk.h", "glu.h")]
CSRC = os.path.join(ROOT, "packed_varlen_rotary_rope_amd", "csrc")

OK, EINVAL, EUNSUPPORTED = 0, -1, -2
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation or is empty


def declared_functions():
    names = []
    for header in HEADERS:
        text = open(header).read()
        names += re.findall(r"^\s*(?:int32_t|const char\*)\s+((?:rope|glu)_\w+)\s*\(", text,
                            re.M)
    return names


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"rope_qk_fwd", "rope_qk_bwd", "rope_qk_apply", "rope_positions",
                          "rope_cos_sin", "rope_inv_freq", "rope_status_str", "rope_abi_version",
                          "glu_fwd", "glu_bwd"}
    out = subprocess.run(["nm", "-D", "--defined-only", rope.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = rope._lib
    for n in names:
        assert hasattr(lib, n)


def test_version_and_status_strings():
    assert rope.abi_version() == 5
    lib = rope._lib
    for st in (0, -1, -2, -3):
        assert lib.rope_status_str(st).decode().startswith("ROPE_")
    assert b"unknown" in lib.rope_status_str(7)


def apply(**kw):
    a = dict(q=FAKE, k=FAKE, T=16, Hq=4, Hkv=2, D=128, cu=FAKE, num_seqs=2, seqused=None,
             theta=1e4, dtype=1, direction=1, index_mode=0, tpw=0, stream=None)
    a.update(kw)
    return rope._lib.rope_qk_apply(a["q"], a["k"], a["T"], a["Hq"], a["Hkv"], a["D"], a["cu"],
                                   a["num_seqs"], a["seqused"], a["theta"], a["dtype"],
                                   a["direction"], a["index_mode"], a["tpw"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(dtype=3), EUNSUPPORTED),
    (dict(dtype=-1), EUNSUPPORTED),
    (dict(T=-1), EINVAL),
    (dict(Hq=-1), EINVAL),
    (dict(Hkv=-2), EINVAL),
    (dict(Hq=5000), EINVAL),
    (dict(Hq=0, Hkv=0), EINVAL),
    (dict(D=127), EINVAL),
    (dict(D=0), EINVAL),
    (dict(D=514), EINVAL),
    (dict(theta=0.5), EINVAL),
    (dict(theta=float("nan")), EINVAL),
    (dict(theta=float("inf")), EINVAL),
    (dict(theta=-1e4), EINVAL),
    (dict(num_seqs=-1), EINVAL),
    (dict(direction=0), EINVAL),
    (dict(direction=2), EINVAL),
    (dict(index_mode=3), EINVAL),
    (dict(tpw=-1), EINVAL),
    (dict(tpw=1025), EINVAL),
    (dict(cu=None), EINVAL),
    (dict(q=None), EINVAL),
    (dict(k=None), EINVAL),
    # Q alone needs 2^31 elements of index space: 32-bit indexing cannot be forced.
    (dict(T=524288, Hq=32, Hkv=8, D=128, index_mode=1), EINVAL),
    # Empty work: valid, and returns before touching the GPU.
    (dict(T=0, q=None, k=None, cu=None), OK),
    (dict(num_seqs=0, cu=None), OK),
])
def test_validation(kw, expect):
    assert apply(**kw) == expect


def apply_ex(**kw):
    a = dict(q=FAKE, k=FAKE, T=16, Hq=4, Hkv=2, D=128, qs=0, ks=0, cu=FAKE, num_seqs=2,
             seqused=None, offsets=None, ids=None, theta=1e4, scale=1.0, dtype=1, direction=1,
             index_mode=0, tpw=0, stream=None)
    a.update(kw)
    return rope._lib.rope_qk_apply_ex(a["q"], a["k"], a["T"], a["Hq"], a["Hkv"], a["D"], a["qs"],
                                      a["ks"], a["cu"], a["num_seqs"], a["seqused"], a["offsets"],
                                      a["ids"], a["theta"], a["scale"], a["dtype"],
                                      a["direction"], a["index_mode"], a["tpw"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(scale=0.5), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL),
    (dict(scale=1e300), EINVAL),  # not finite once rounded to fp32
    (dict(scale=-4.0), EINVAL),
    (dict(cu=None, ids=None), EINVAL),
    (dict(ids=FAKE, theta=0.0), EINVAL),
    (dict(ids=FAKE, D=3), EINVAL),
    (dict(ids=FAKE, q=None), EINVAL),
    (dict(dtype=9, ids=FAKE), EUNSUPPORTED),
    (dict(T=0, q=None, k=None, cu=None, ids=None), OK),
    (dict(num_seqs=0, cu=None), OK),
    (dict(qs=-1), EINVAL),
    (dict(qs=4 * 128 - 1), EINVAL),             # consecutive q tokens would overlap
    (dict(ks=2 * 128 - 2), EINVAL),
    (dict(qs=1 << 45), EINVAL),                 # 16 tokens span 2^49 elements
    (dict(ks=1 << 45), EINVAL),
    (dict(qs=1 << 28, index_mode=1), EINVAL),   # 32-bit offsets asked for, 64 needed
    (dict(Hq=0, q=None, qs=-1), EINVAL),
])
def test_validation_ex(kw, expect):
    assert apply_ex(**kw) == expect


def apply_table(**kw):
    a = dict(q=FAKE, k=FAKE, T=16, Hq=4, Hkv=2, D=128, qs=0, ks=0, cu=FAKE, num_seqs=2,
             seqused=None, offsets=None, ids=None, ct=FAKE, st=FAKE, rows=8, dtype=1,
             direction=1, index_mode=0, tpw=0, stream=None)
    a.update(kw)
    return rope._lib.rope_qk_apply_table(a["q"], a["k"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                         a["qs"], a["ks"], a["cu"], a["num_seqs"], a["seqused"],
                                         a["offsets"], a["ids"], a["ct"], a["st"], a["rows"],
                                         a["dtype"], a["direction"], a["index_mode"], a["tpw"],
                                         a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(ct=None), EINVAL),
    (dict(st=None), EINVAL),
    (dict(ct=None, st=None, T=0, q=None, k=None), EINVAL),  # tables are always required
    (dict(rows=0), EINVAL),
    (dict(rows=-5), EINVAL),
    (dict(dtype=5), EUNSUPPORTED),
    (dict(dtype=5, ct=None), EUNSUPPORTED),
    (dict(D=130 + 1), EINVAL),
    (dict(direction=0), EINVAL),
    (dict(cu=None, ids=None), EINVAL),
    (dict(q=None), EINVAL),
    (dict(qs=4 * 128 - 1), EINVAL),
    (dict(T=0, q=None, k=None, cu=None), OK),
    (dict(num_seqs=0, cu=None), OK),
])
def test_validation_table(kw, expect):
    """The table entry point validates like rope_qk_apply_ex, plus its tables; it has
    no theta or scale to check."""
    assert apply_table(**kw) == expect


def apply_padded(**kw):
    a = dict(q=FAKE, k=FAKE, T=16, Hq=4, Hkv=2, D=128, qs=0, ks=0, cu=FAKE, num_seqs=2,
             seqused=FAKE, cv=FAKE, valid=10, offsets=None, theta=1e4, scale=1.0, dtype=1,
             direction=1, index_mode=0, stream=None)
    a.update(kw)
    return rope._lib.rope_qk_apply_padded(a["q"], a["k"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                          a["qs"], a["ks"], a["cu"], a["num_seqs"],
                                          a["seqused"], a["cv"], a["valid"], a["offsets"],
                                          a["theta"], a["scale"], a["dtype"], a["direction"],
                                          a["index_mode"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(valid=-1), EINVAL),
    (dict(valid=17), EINVAL),                   # more rotated tokens than rows
    (dict(cv=None), EINVAL),
    (dict(dtype=4), EUNSUPPORTED),
    (dict(theta=0.5), EINVAL),
    (dict(scale=0.5), EINVAL),
    (dict(D=127), EINVAL),
    (dict(direction=0), EINVAL),
    (dict(index_mode=3), EINVAL),
    (dict(cu=None), EINVAL),
    (dict(q=None), EINVAL),
    (dict(qs=4 * 128 - 1), EINVAL),
    (dict(T=524288, Hq=32, Hkv=8, D=128, index_mode=1, valid=100), EINVAL),
    # Empty work: valid, and returns before touching the GPU.
    (dict(valid=0, cv=None), OK),
    (dict(num_seqs=0, cu=None, cv=None), OK),
    (dict(T=0, q=None, k=None, cu=None, cv=None, valid=0), OK),
])
def test_validation_padded(kw, expect):
    """The compact padded entry point validates like rope_qk_apply_ex, plus its
    rotated-token count (0..T) and its cu_valid array."""
    assert apply_padded(**kw) == expect


def test_valid_prefix_validation():
    lib = rope._lib
    assert lib.rope_valid_prefix(FAKE, -1, None, FAKE, None) == EINVAL
    assert lib.rope_valid_prefix(FAKE, 2**31 - 1, None, FAKE, None) == EINVAL
    assert lib.rope_valid_prefix(FAKE, 2, None, None, None) == EINVAL
    assert lib.rope_valid_prefix(None, 2, FAKE, FAKE, None) == EINVAL


def test_fwd_bwd_positions_cos_sin_validation():
    lib = rope._lib
    args = (FAKE, FAKE, 16, 4, 2, 127, FAKE, 2, None, 1e4, 1, None)
    assert lib.rope_qk_fwd(*args) == EINVAL
    assert lib.rope_qk_bwd(*args) == EINVAL
    assert lib.rope_positions(FAKE, -1, None, 16, FAKE, FAKE, None) == EINVAL
    assert lib.rope_positions(None, 2, None, 16, FAKE, FAKE, None) == EINVAL
    assert lib.rope_positions(FAKE, 2, None, -5, FAKE, FAKE, None) == EINVAL
    assert lib.rope_positions(FAKE, 2, None, 0, FAKE, FAKE, None) == OK
    assert lib.rope_cos_sin(4, 7, 1e4, FAKE, FAKE, None) == EINVAL  # odd D
    assert lib.rope_cos_sin(-1, 8, 1e4, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin(4, 8, 0.5, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin(4, 8, 1e4, None, FAKE, None) == EINVAL
    assert lib.rope_cos_sin(4, 8, 1e4, FAKE, None, None) == EINVAL
    assert lib.rope_cos_sin(0, 8, 1e4, None, None, None) == OK
    assert lib.rope_cos_sin_at(FAKE, 4, 7, 1e4, 1.0, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin_at(FAKE, -1, 8, 1e4, 1.0, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin_at(None, 4, 8, 1e4, 1.0, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin_at(FAKE, 0, 8, 1e4, 1.0, FAKE, FAKE, None) == OK
    assert lib.rope_inv_freq(1e4, 8, None) == EINVAL
    assert lib.rope_qk_fwd_pos(FAKE, FAKE, 16, 4, 2, 128, None, 1e4, 1, None) == EINVAL
    assert lib.rope_qk_bwd_pos(FAKE, FAKE, 16, 4, 2, 127, FAKE, 1e4, 1, None) == EINVAL
    assert lib.rope_qk_fwd_pos(None, None, 0, 4, 2, 128, None, 1e4, 1, None) == OK
    assert lib.rope_positions_ex(None, 2, None, None, None, 16, FAKE, FAKE, None) == EINVAL
    assert lib.rope_positions_ex(None, 0, None, None, None, 0, FAKE, FAKE, None) == OK
    assert lib.rope_cos_sin_at(FAKE, 4, 8, 1e4, 0.9, FAKE, FAKE, None) == EINVAL
    assert lib.rope_cos_sin_at(FAKE, 0, 8, 1e4, 2.0, FAKE, FAKE, None) == OK


@pytest.mark.parametrize("theta,D", [(1e4, 16), (1e6, 128), (1e4, 128), (5e5, 64), (1e6, 80),
                                     (1.0, 4), (1e6, 512)])
def test_host_inv_freq(theta, D):
    got = rope.inv_freq(theta, D).numpy()
    ref = ref_inv_freq(theta, D)  # theta^(-2j/D) to 200 bits, rounded once to fp32
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(got.view(np.uint32), oracle.inv_freq(theta, D).view(np.uint32))


def test_host_inv_freq_many_thetas():
    """The fast host path (double pow, extended precision only near a binary32
    midpoint) against the oracle (extended precision throughout, itself pinned to
    mpmath) for 300 random log-uniform theta in [1, 1e12] and every even D up to 512
    in turn, and against mpmath directly on a sample."""
    rng = np.random.default_rng(44)
    thetas = np.concatenate([[1.0, 2.0, 1e4, 5e5, 1e6, 1e7, 8e6, 2.5e5, 1e12],
                             10.0 ** rng.uniform(0, 12, 300)])
    Ds = list(range(2, 514, 2))
    for i, theta in enumerate(thetas):
        D = Ds[i % len(Ds)] if i >= 9 else 128
        got = rope.inv_freq(float(theta), D).numpy()
        assert np.array_equal(got.view(np.uint32), oracle.inv_freq(float(theta), D).view(np.uint32)), \
            (theta, D)
        if i % 30 == 0:
            assert np.array_equal(got.view(np.uint32), ref_inv_freq(float(theta), D).view(np.uint32))


def test_trig_constants_regenerate():
    sys.path.insert(0, CSRC)
    try:
        import gen_trig_constants as gen
    finally:
        sys.path.remove(CSRC)
    assert open(os.path.join(CSRC, "trig_constants.h")).read() == gen.render()
    # Independent check of the pi/2 split against mpmath's pi.
    src = open(os.path.join(CSRC, "trig_constants.h")).read()
    parts = [float(re.search(r"PIO2_%d = ([^;]+);" % i, src).group(1)) for i in (1, 2, 3)]
    mpmath.mp.prec = 300
    err = sum(mpmath.mpf(p) for p in parts) - mpmath.pi / 2
    assert abs(err) < mpmath.mpf(2) ** -150


def test_glu_constants_regenerate():
    """glu_constants.h is what its generator writes; the roots it holds are roots of
    the derivatives written independently here (mpmath, literal definitions)."""
    sys.path.insert(0, CSRC)
    try:
        import gen_glu_constants as gen
    finally:
        sys.path.remove(CSRC)
    text = open(os.path.join(CSRC, "glu_constants.h")).read()
    assert text == gen.generate()
    mpmath.mp.dps = 40

    def silu(x):
        return x / (1 + mpmath.exp(-x))

    def gelu(x):
        return x * (1 + mpmath.erf(x / mpmath.sqrt(2))) / 2

    def gelu_tanh(x):
        k = mpmath.sqrt(2 / mpmath.pi)
        return x / 2 * (1 + mpmath.tanh(k * (x + mpmath.mpf("0.044715") * x ** 3)))

    for name, f in (("Silu", silu), ("Gelu", gelu), ("GeluTanh", gelu_tanh)):
        # the literals are fp32 values: round the parsed decimal back to fp32
        hi = float(np.float32(re.search(r"k%sRootHi = ([^f]+)f;" % name, text).group(1)))
        lo = float(np.float32(re.search(r"k%sRootLo = ([^f]+)f;" % name, text).group(1)))
        root = mpmath.mpf(hi) + mpmath.mpf(lo)
        slope = mpmath.diff(f, root, 2)
        assert abs(mpmath.diff(f, root) / slope) < 1e-13, name  # |root error| < 1e-13


def test_token_stride_of_views():
    """Token strides the binding derives from [T, H, D] views (host-only logic)."""
    T, Hq, Hkv, D = 5, 4, 2, 8
    qkv = torch.zeros(T, (Hq + 2 * Hkv) * D)
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].view(T, Hkv, D)
    assert rope._token_stride(q, "q") == (Hq + 2 * Hkv) * D
    assert rope._token_stride(k, "k") == (Hq + 2 * Hkv) * D
    assert rope._token_stride(torch.zeros(T, Hq, D), "q") == 0
    assert rope._token_stride(q[:1], "q") == 0          # one token: stride unused
    with pytest.raises(ValueError):
        rope._token_stride(torch.zeros(T, D, Hq).transpose(1, 2), "q")
    with pytest.raises(ValueError):
        rope._token_stride(torch.zeros(T, Hq, 2 * D)[:, :, ::2], "q")


# ---------------------------------------------------------------- SwiGLU / GeGLU validation

def glu(bwd=False, **kw):
    a = dict(kind=0, dh=FAKE, e=FAKE, g=FAKE, out0=FAKE, out1=FAKE, rows=16, cols=64, ins=0,
             outs=0, dtype=1, index_mode=0, stream=None)
    a.update(kw)
    if bwd:
        return rope._lib.glu_bwd(a["kind"], a["dh"], a["e"], a["g"], a["out0"], a["out1"],
                                 a["rows"], a["cols"], a["ins"], a["outs"], a["dtype"],
                                 a["index_mode"], a["stream"])
    return rope._lib.glu_fwd(a["kind"], a["e"], a["g"], a["out0"], a["rows"], a["cols"], a["ins"],
                             a["outs"], a["dtype"], a["index_mode"], a["stream"])


@pytest.mark.parametrize("bwd", [False, True])
@pytest.mark.parametrize("kw,expect", [
    (dict(kind=3), EINVAL),
    (dict(kind=-1), EINVAL),
    (dict(dtype=5), EUNSUPPORTED),
    (dict(rows=-1), EINVAL),
    (dict(cols=-1), EINVAL),
    (dict(ins=63), EINVAL),                       # rows would overlap
    (dict(outs=10), EINVAL),
    (dict(ins=-64), EINVAL),
    (dict(e=None), EINVAL),
    (dict(g=None), EINVAL),
    (dict(out0=None), EINVAL),
    (dict(index_mode=3), EINVAL),
    (dict(rows=1 << 20, ins=1 << 29), EINVAL),    # span 2^49 elements
    (dict(rows=1 << 16, cols=1 << 16, index_mode=1), EINVAL),  # 2^32 elements need 64 bits
    (dict(rows=0), OK),
    (dict(cols=0), OK),
    (dict(rows=0, e=None, g=None, out0=None, out1=None, dh=None), OK),
])
def test_glu_validation(bwd, kw, expect):
    assert glu(bwd, **kw) == expect


def test_glu_bwd_needs_its_extra_pointers():
    assert glu(True, dh=None) == EINVAL
    assert glu(True, out1=None) == EINVAL


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the package refuses to import: there is no CPU
    fallback. A copy of the package without its .so is imported in a subprocess."""
    import shutil
    pkg = os.path.join(ROOT, "packed_varlen_rotary_rope_amd")
    dst = tmp_path / "packed_varlen_rotary_rope_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    assert not any(p.suffix == ".so" for p in dst.iterdir())
    r = subprocess.run([sys.executable, "-c", "import packed_varlen_rotary_rope_amd"],
                       cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "no fallback" in r.stderr.lower()


def test_build_entry_loads_builder_without_library(tmp_path):
    """A fresh checkout has no library yet: the build entry point must reach the
    builder without importing the package (whose import needs the library)."""
    import shutil
    pkg = os.path.join(ROOT, "packed_varlen_rotary_rope_amd")
    shutil.copytree(pkg, tmp_path / "packed_varlen_rotary_rope_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path)
    code = ("import sys, __graft_entry__ as g; m = g._load_lib_builder(); "
            "assert 'packed_varlen_rotary_rope_amd' not in sys.modules; "
            "print(m.ARCH, len(m.SRCS))")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["gfx950", "2"]


FAST_DIV_CHECK = r"""
#include <stdio.h>
#include <stdlib.h>
#include "fast_div.h"
using namespace fastdiv;
static uint64_t state = 88172645463325252ull;
static uint32_t rnd(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return (uint32_t)state; }
static int check(uint32_t n, uint32_t d, FastDiv f) {
  if (div(n, f) != n / d) { printf("n=%u d=%u got %u\n", n, d, div(n, f)); return 1; }
  return 0;
}
int main(void) {
  const uint32_t top = (1u << kMaxDividendBits) - 1;
  int bad = 0;
  /* every divisor a launch can have (row groups per token <= 2 * 4096), near every
     multiple of d that the edges of the range hold, and at random */
  for (uint32_t d = 1; d <= 8192 && !bad; ++d) {
    const FastDiv f = make(d);
    if (f.mul == 0) return 2;
    for (uint32_t j = 0; j < 64; ++j) {
      const uint64_t m = (uint64_t)j * d, m2 = (uint64_t)(top / d - j) * d;
      for (int e = -1; e <= 1; ++e) {
        if ((int64_t)m + e >= 0 && m + e <= top) bad |= check((uint32_t)(m + e), d, f);
        if ((int64_t)m2 + e >= 0 && m2 + e <= top) bad |= check((uint32_t)(m2 + e), d, f);
      }
    }
    for (int i = 0; i < 2000; ++i) bad |= check(rnd() & top, d, f);
  }
  /* exhaustively for a few divisors, and for large ones at random */
  const uint32_t some[] = {3, 5, 7, 9, 10, 17, 40, 72, 4097};
  for (uint32_t d : some) {
    const FastDiv f = make(d);
    for (uint32_t n = 0; n <= top && !bad; ++n) bad |= check(n, d, f);
  }
  for (int i = 0; i < 200000 && !bad; ++i) {
    const uint32_t d = 1 + (rnd() & 0x7ffffffe);
    bad |= check(rnd() & top, d, make(d));
  }
  printf(bad ? "FAIL\n" : "ok\n");
  return bad;
}
"""


def test_fast_division_constants(tmp_path):
    """The row-group kernel maps a workgroup index to (token, row group) as
    (n * mul) >> shift with host-made constants (fastdiv::make): equal to n / d for
    every divisor a launch can have, checked near range edges, at random and
    exhaustively over all n < 2^26 for a few divisors."""
    src = tmp_path / "fast_div_check.cpp"
    src.write_text(FAST_DIV_CHECK)
    exe = tmp_path / "fast_div_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
