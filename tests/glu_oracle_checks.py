"""Pins for the SwiGLU / GeGLU CPU oracle: each check ties it to something other
than itself -- the literal textbook definitions evaluated by mpmath at high
precision (including the forms with 1 + erf and 1 + tanh that the oracle avoids),
numerical derivatives of those definitions, torch's float64 activations and
autograd, symmetry identities, printed values of the normal CDF, and exact
rational rounding.

Every check takes an ``oracle.glu.GluOracle`` handle so that the mutation test
can run the same checks against deliberately broken builds (on the CPU).

Page cited: Unsloth, "Entrainement des LLM 3 fois plus rapide avec les noyaux
Unsloth + le packing" (opening list and section "Indexage int64 pour les
kernels Triton"), which names the SwiGLU and GeGLU kernels; the formulas are the
standard ones (Shazeer 2020; Hendrycks & Gimpel 2016).
"""
from __future__ import annotations

import math
from fractions import Fraction

import mpmath
import numpy as np
import torch

KINDS = ("swiglu", "geglu", "geglu_tanh")
GRID = np.concatenate([np.linspace(-30.0, 30.0, 241),
                       [-100.0, -90.0, -88.5, -50.0, -12.0, -1e-3, 0.0, 1e-3, 1.0,
                        math.log(3.0), 5.0, 50.0, 100.0, -0.7517915, -1.2784645]])


# ---------------------------------------------------------------- literal definitions

def mp_act(kind: str, e):
    """The literal definitions, with the working precision raised until the sums
    1 + erf(x) and 1 + tanh(u) resolve their negative tails (about |x|^2/ln 10 and
    2|u|/ln 10 digits). Past 3000 digits the tanh form uses the exact identity
    1 + tanh(u) = 2 / (1 + exp(-2u)); no grid point below needs it."""
    e = mpmath.mpf(e)
    if kind == "swiglu":
        return e / (1 + mpmath.exp(-e))
    if kind == "geglu":
        digits = 40 + (int(float(e * e) / 2 / 2.3) if e < 0 else 0)
        with mpmath.workdps(max(mpmath.mp.dps, digits)):
            return e * (1 + mpmath.erf(e / mpmath.sqrt(2))) / 2
    with mpmath.workdps(max(mpmath.mp.dps, 40)):
        u = mpmath.sqrt(2 / mpmath.pi) * (e + mpmath.mpf("0.044715") * e ** 3)
    digits = 40 + (int(2 * abs(float(u)) / 2.3) if e < 0 else 0)
    with mpmath.workdps(max(mpmath.mp.dps, min(digits, 3000))):
        if digits > 3000:
            return e / (1 + mpmath.exp(-2 * u))
        return e / 2 * (1 + mpmath.tanh(u))


def torch_act(kind: str, x: torch.Tensor) -> torch.Tensor:
    if kind == "swiglu":
        return torch.nn.functional.silu(x)
    return torch.nn.functional.gelu(x, approximate="none" if kind == "geglu" else "tanh")


def bf16_words(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def words_to_f64(words: np.ndarray, dtype: str) -> np.ndarray:
    """Decode storage words with torch's own conversion (independent of the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.double().numpy()


# ---------------------------------------------------------------- activations

def check_act_mpmath(o):
    """act(e) against the literal definitions at 120 digits (1 + erf and 1 + tanh
    evaluated as written: enough digits make the cancellation harmless)."""
    with mpmath.workdps(120):
        for kind in KINDS:
            got = o.act(kind, GRID)
            for e, g in zip(GRID, got):
                ref = mp_act(kind, e)
                tol = mpmath.mpf(1e-14) * (1 + e * e) * abs(ref) + mpmath.mpf(1e-300)
                assert abs(mpmath.mpf(g) - ref) <= tol, (kind, e, g, ref)


def check_grad_mpmath(o):
    """act'(e) against a numerical derivative of the literal definition."""
    with mpmath.workdps(60):
        for kind in KINDS:
            pts = GRID[np.abs(GRID) <= (50 if kind == "swiglu" else 20)]
            got = o.grad(kind, pts)
            for e, g in zip(pts, got):
                ref = mpmath.diff(lambda x: mp_act(kind, x), mpmath.mpf(e))
                tol = mpmath.mpf(1e-12) * abs(ref) + mpmath.mpf(1e-15)
                assert abs(mpmath.mpf(g) - ref) <= tol, (kind, e, g, ref)


def check_symmetry(o):
    """act(x) - act(-x) = x and act'(x) + act'(-x) = 1: Phi(x) + Phi(-x) = 1,
    sigmoid(x) + sigmoid(-x) = 1, and tanh is odd."""
    x = np.concatenate([np.geomspace(1e-3, 12.0, 60)])
    for kind in KINDS:
        d = o.act(kind, x) - o.act(kind, -x)
        assert np.all(np.abs(d - x) <= 1e-14 * x), kind
        s = o.grad(kind, x) + o.grad(kind, -x)
        assert np.all(np.abs(s - 1.0) <= 1e-13 * (1 + x * x)), kind


def check_hand_values(o):
    """silu(ln 3) = (3/4) ln 3, since sigmoid(ln 3) = 1/(1 + 1/3); gelu(+-1) =
    +-Phi(+-1) from the normal table (0.8413447460685429, 0.15865525393145707);
    all three activations are 0 at 0 with slope 1/2."""
    ln3 = math.log(3.0)
    assert abs(o.act("swiglu", [ln3])[0] - 0.75 * ln3) <= 2e-16 * ln3
    assert abs(o.act("geglu", [1.0])[0] - 0.8413447460685429) <= 2e-16
    assert abs(o.act("geglu", [-1.0])[0] + 0.15865525393145707) <= 2e-16
    for kind in KINDS:
        assert o.act(kind, [0.0])[0] == 0.0
        assert o.grad(kind, [0.0])[0] == 0.5


def check_torch_float64(o):
    """Forward values and autograd gradients from torch's float64 silu / gelu /
    gelu(tanh) on moderate inputs (|e| <= 3, where torch's 1 + erf and 1 + tanh
    lose at most ~1e-13 to cancellation), through the array entry points with f32
    storage (values exact on both sides)."""
    rng = np.random.default_rng(11)
    rows, cols = 7, 33
    e = np.clip(rng.standard_normal((rows, cols)), -3, 3).astype(np.float32)
    g = rng.standard_normal((rows, cols)).astype(np.float32)
    dh = rng.standard_normal((rows, cols)).astype(np.float32)
    for kind in KINDS:
        et = torch.tensor(e, dtype=torch.float64, requires_grad=True)
        gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
        h = torch_act(kind, et) * gt
        h.backward(torch.tensor(dh, dtype=torch.float64))
        got_h = o.fwd(kind, e, g, "f32")
        assert np.allclose(got_h, h.detach().numpy(), rtol=1e-12, atol=1e-15), kind
        de, dg = o.bwd(kind, dh, e, g, "f32")
        scale = np.abs(dh.astype(np.float64) * g)
        assert np.all(np.abs(de - et.grad.numpy()) <= 1e-12 * scale + 1e-15), kind
        assert np.allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-15), kind


def check_arrays_strided_16bit(o):
    """bf16 and f16 storage, e and g rows 11 elements apart and dh rows 13 apart,
    NaN in every gap: element-wise equal (to 1e-12) to torch float64 on
    torch-decoded values, and no gap element is ever read."""
    rng = np.random.default_rng(12)
    rows, cols, stride, dh_stride = 5, 7, 11, 13
    for dtype in ("bf16", "f16"):
        def words(x):
            if dtype == "bf16":
                return bf16_words(x)
            return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)
        nan = words(np.full(1, np.nan))[0]
        bufs = {}
        for name in ("e", "g", "dh"):
            vals = rng.standard_normal((rows, cols)) * (2.5 if name == "e" else 1.0)
            buf = np.full((rows, dh_stride if name == "dh" else stride), nan, dtype=np.uint16)
            buf[:, :cols] = words(vals)
            bufs[name] = buf
        e_v, g_v, dh_d = (bufs[n][:, :cols] for n in ("e", "g", "dh"))
        ev, gv, dv = (words_to_f64(np.ascontiguousarray(a), dtype) for a in (e_v, g_v, dh_d))
        for kind in KINDS:
            et = torch.tensor(ev, requires_grad=True)
            gt = torch.tensor(gv, requires_grad=True)
            h = torch_act(kind, et) * gt
            h.backward(torch.tensor(dv))
            got = o.fwd(kind, e_v, g_v, dtype)
            assert np.all(np.isfinite(got)), (kind, dtype)
            assert np.allclose(got, h.detach().numpy(), rtol=1e-12, atol=1e-15), (kind, dtype)
            de, dg = o.bwd(kind, dh_d, e_v, g_v, dtype)
            scale = np.abs(dv * gv)
            assert np.all(np.abs(de - et.grad.numpy()) <= 1e-12 * scale + 1e-15), (kind, dtype)
            assert np.allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-15), (kind, dtype)


def check_f16_decode_extremes(o):
    """f16 decoding over every 37th finite f16 word (subnormals and the largest
    values included) through the array entry point: gelu_tanh(e) * 1 with e = each
    word, against mpmath on the values torch decodes from the same words."""
    words = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (words & 0x7C00) != 0x7C00
    w = np.ascontiguousarray(words[finite][::37]).reshape(1, -1)
    ones = np.full_like(w, np.float16(1.0).view(np.uint16))
    got = o.fwd("geglu_tanh", w, ones, "f16")[0]
    vals = words_to_f64(w[0], "f16")
    with mpmath.workdps(40):
        for v, g in zip(vals, got):
            ref = mp_act("geglu_tanh", v)
            assert abs(mpmath.mpf(g) - ref) <= mpmath.mpf(1e-13) * (1 + v * v) * abs(ref) \
                + mpmath.mpf(1e-300), (v, g)


# ---------------------------------------------------------------- rounding

def _nearest(exact: Fraction, cands):
    """Nearest candidate value to exact; ties go to the candidate with an even last bit."""
    best = None
    for bits, val in cands:
        d = abs(Fraction(val) - exact) if math.isfinite(val) else None
        if d is None:
            continue
        key = (d, bits & 1)
        if best is None or key < best[0]:
            best = (key, bits, val)
    return best[1], best[2]


def check_round(o):
    """One rounding from double to f32 / bf16 / f16 against exhaustive search among
    neighbouring representable values with exact rationals (ties to even), on
    random doubles, exact ties, subnormals and the overflow edges."""
    rng = np.random.default_rng(13)
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-8, 8, 300))
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
           1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -25,
           5 * 2.0 ** -26, 1e-40, -7e-39, 65519.0, 65520.0, 70000.0, 3.3e38, 3.39e38, -1e39]
    xs = np.array(xs, dtype=np.float64)
    # f32
    got = o.round("f32", xs)
    for x, g in zip(xs, got):
        with np.errstate(over="ignore"):
            f = np.float32(x)  # numpy's double -> float is a single correct rounding
        assert g.view(np.uint32) == f.view(np.uint32), (x, g, f)
    # f16: numpy's double -> half is a single correct rounding too; check both ways
    got = o.round("f16", xs)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    # bf16: exhaustive among the three words around the truncated float32 pattern
    got = o.round("bf16", xs)
    for x, g in zip(xs, got):
        if abs(x) >= 3.3961776e38:  # at or past the rounding boundary to infinity
            assert g & 0x7FFF == 0x7F80, x
            continue
        t = int(np.float32(x).view(np.uint32)) >> 16
        cands = []
        for b in (t - 1, t, t + 1):
            b &= 0xFFFF
            val = float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
            cands.append((b, val))
        bits, _ = _nearest(Fraction(float(x)), cands)
        assert int(g) == bits, (x, hex(int(g)), hex(bits))


# Cheap checks first: the mutation test stops at the first failing check.
ALL_CHECKS = [
    check_round,
    check_hand_values,
    check_symmetry,
    check_torch_float64,
    check_arrays_strided_16bit,
    check_grad_mpmath,
    check_act_mpmath,
    check_f16_decode_extremes,
]
