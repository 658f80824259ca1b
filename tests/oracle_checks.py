"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- a closed form, an arbitrary-precision value (mpmath), the block
rotation matrix R as the Unsloth page defines it (tests/golden), complex
multiplication, invariants of a rotation, exact rational arithmetic, brute
force on tiny inputs, or torch's bf16 cast.

Every check takes an ``oracle.Oracle`` handle so that the mutation test can run
the same checks against deliberately broken builds of the oracle (on the CPU)
and show that each plausible mistake fails at least one of them.

Page cited throughout: Unsloth, "Entrainement des LLM 3 fois plus rapide avec
les noyaux Unsloth + le packing" (sections "Kernel Triton QK RoPE fusionne avec
packing" and "Packing non contamine").
"""
from __future__ import annotations

import cmath
import math
import os
from fractions import Fraction

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

mpmath.mp.prec = 200


# ---------------------------------------------------------------------------- helpers

def rn_f32(v) -> np.float32:
    """Correctly rounded float32 of an exact value (Fraction or mpmath mpf); ties to even."""
    exact = Fraction(v) if not isinstance(v, mpmath.mpf) else v
    f = np.float32(float(v))
    best, best_d = None, None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        cv = Fraction(float(c)) if isinstance(exact, Fraction) else mpmath.mpf(float(c))
        d = abs(cv - exact)
        if best is None or d < best_d or (d == best_d and int(np.float32(c).view(np.uint32)) % 2 == 0):
            best, best_d = np.float32(c), d
    return best


def ref_inv_freq(theta: float, D: int) -> np.ndarray:
    """theta^(-2j/D) to 200 bits, correctly rounded to fp32."""
    th = mpmath.mpf(theta)
    return np.array([rn_f32(th ** (-mpmath.mpf(2 * j) / D)) for j in range(D // 2)],
                    dtype=np.float32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def random_bf16(rng, shape) -> np.ndarray:
    """Random N(0,1) values as bf16 bits (via torch's RNE cast)."""
    import torch
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def load_golden_matrices():
    mats, cur, rows = {}, None, []
    with open(os.path.join(GOLDEN, "rotation_matrix_R.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line[0].isalpha():
                if cur:
                    mats[cur] = np.array(rows, dtype=np.float64)
                name, d = line.split()
                cur, rows = (name, int(d.split("=")[1])), []
            else:
                rows.append([float(v) for v in line.split()])
    mats[cur] = np.array(rows, dtype=np.float64)
    return mats


def full_cos_sin(c_half: np.ndarray, s_half: np.ndarray):
    """cos/sin of the D/2 frequencies laid out over D elements (j and j + D/2 share)."""
    return np.concatenate([c_half, c_half], -1), np.concatenate([s_half, s_half], -1)


# ---------------------------------------------------------------------------- checks

def check_inv_freq_closed_form(o):
    # theta^0 = 1 for every theta; theta = 1e4, D = 4 gives [1, 1e4^(-1/2)] = [1, 0.01].
    f = o.inv_freq(1e4, 4)
    assert f.tolist() == [1.0, float(np.float32(0.01))], f
    for theta in (2.0, 1e4, 5e5, 1e6):
        for D in (2, 16, 64, 128):
            assert o.inv_freq(theta, D)[0] == 1.0
    # D = 16, theta = 1e4: the exponents -2j/16 give 10^(-j/2).
    f = o.inv_freq(1e4, 16)
    ref = [np.float32(10.0 ** (-j / 2)) for j in range(8)]
    assert np.array_equal(f, np.array(ref, dtype=np.float32)), (f, ref)


def check_inv_freq_mpmath(o):
    for theta, D in ((1e4, 16), (1e6, 128), (1e4, 128), (5e5, 64), (1e6, 80), (1e6, 2)):
        got = o.inv_freq(theta, D)
        ref = ref_inv_freq(theta, D)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (theta, D, got, ref)


def check_cos_sin_pos0(o):
    c, s = o.cos_sin([0], 128, 1e6)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    assert not np.any(np.signbit(s))


def check_cos_sin_mpmath(o):
    rng = np.random.default_rng(7)
    cases = [
        (1e4, 16, [0, 1, 2, 3, 38, 63]),
        (1e6, 128, [1, 100, 4095, 16383, 32767, 524287] + rng.integers(0, 524288, 10).tolist()),
    ]
    for theta, D, plist in cases:
        f = ref_inv_freq(theta, D)
        c, s = o.cos_sin(plist, D, theta)
        for i, p in enumerate(plist):
            for j in range(D // 2):
                angle = np.float32(np.float32(p) * f[j])  # one fp32 multiply
                a = mpmath.mpf(float(angle))
                assert c[i, j] == rn_f32(mpmath.cos(a)), (theta, D, p, j, c[i, j])
                assert s[i, j] == rn_f32(mpmath.sin(a)), (theta, D, p, j, s[i, j])


def check_block_matrix_R(o):
    """Forward = x*cos + (x @ R)*sin, backward = x*cos + (x @ R^T)*sin, R from the page."""
    mats = load_golden_matrices()
    rng = np.random.default_rng(11)
    for D in (4, 6, 16):
        if D in (4, 6):
            R, RT = mats[("R", D)], mats[("RT", D)]
        else:  # the same block rule, built with numpy
            I, Z = np.eye(D // 2), np.zeros((D // 2, D // 2))
            R, RT = np.block([[Z, I], [-I, Z]]), np.block([[Z, -I], [I, Z]])
        assert np.array_equal(RT, R.T) and np.array_equal(RT, -R)
        T, H = 9, 3
        theta = 1e4
        x = rng.standard_normal((T, H, D)).astype(np.float32)
        cu = [0, 4, 9]
        pos = [0, 1, 2, 3, 0, 1, 2, 3, 4]
        c_half, s_half = o.cos_sin(pos, D, theta)
        C, S = full_cos_sin(c_half.astype(np.float64), s_half.astype(np.float64))
        xd = x.astype(np.float64)
        for direction, M in ((1, R), (-1, RT)):
            ref = (xd * C[:, None, :] + (xd @ M) * S[:, None, :]).astype(np.float32)
            got = o.rope(x, cu, theta, direction)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (D, direction)


def check_complex_form(o):
    """Each (j, j + D/2) pair is the complex number x_j + i x_{j+D/2} times e^{i angle}."""
    rng = np.random.default_rng(12)
    D, H = 16, 2
    cu = np.array([0, 3, 10, 10, 21], dtype=np.int32)
    T = 21
    pos = np.array([0, 1, 2] + list(range(7)) + list(range(11)))
    c_half, s_half = o.cos_sin(pos, D, 1e4)
    for dtype in ("f32", "bf16"):
        if dtype == "f32":
            x = rng.standard_normal((T, H, D)).astype(np.float32)
            xv = x.astype(np.float64)
        else:
            x = random_bf16(rng, (T, H, D))
            xv = bf16_bits_to_f32(x).astype(np.float64)
        for direction in (1, -1):
            z = xv[..., : D // 2] + 1j * xv[..., D // 2:]
            e = c_half.astype(np.float64) + 1j * direction * s_half.astype(np.float64)
            w = z * e[:, None, :]
            ref = np.concatenate([w.real, w.imag], -1).astype(np.float32)
            got = o.rope(x, cu, 1e4, direction, dtype)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (dtype, direction)


def check_hand_values(o):
    # D = 2: one complex rotation by the angle pos * theta^0 = pos.
    x = np.zeros((4, 1, 2), dtype=np.float32)
    x[3, 0] = [1.0, 2.0]
    y = o.rope(x, [0, 4], 1e4)
    w = (1 + 2j) * cmath.exp(3j)
    assert abs(y[3, 0, 0] - w.real) < 1e-6 and abs(y[3, 0, 1] - w.imag) < 1e-6, (y[3, 0], w)
    # D = 4, theta = 1e4, basis vector e0 at position 1: [cos 1, 0, sin 1, 0].
    x = np.zeros((101, 1, 4), dtype=np.float32)
    x[1, 0, 0] = 1.0
    x[100, 0, 1] = 1.0
    y = o.rope(x, [0, 101], 1e4)
    c1, s1 = np.float32(math.cos(1.0)), np.float32(math.sin(1.0))
    assert y[1, 0].tolist() == [c1, 0.0, s1, 0.0], y[1, 0]
    # e1 at position 100: fp32(100 * fp32(0.01)) is exactly 1.0, so the angle is 1.
    assert np.float32(np.float32(100.0) * np.float32(0.01)) == np.float32(1.0)
    assert y[100, 0].tolist() == [0.0, c1, 0.0, s1], y[100, 0]


def check_identity_at_pos0(o):
    rng = np.random.default_rng(13)
    T = 12
    cu = np.arange(T + 1, dtype=np.int32)  # every sequence has length 1: all positions 0
    for dtype in ("f32", "bf16"):
        x = (rng.standard_normal((T, 3, 8)).astype(np.float32) if dtype == "f32"
             else random_bf16(rng, (T, 3, 8)))
        xf = x if dtype == "f32" else bf16_bits_to_f32(x)
        for theta in (1.5, 1e4, 1e6, 1e12):
            for direction in (1, -1):
                y = o.rope(x, cu, theta, direction, dtype)
                assert np.array_equal(y.view(np.uint32), xf.view(np.uint32))


def check_pair_norm(o):
    rng = np.random.default_rng(14)
    D = 32
    x = rng.standard_normal((300, 2, D)).astype(np.float32)
    y = o.rope(x, [0, 300], 1e4).astype(np.float64)
    xd = x.astype(np.float64)
    nx = xd[..., : D // 2] ** 2 + xd[..., D // 2:] ** 2
    ny = y[..., : D // 2] ** 2 + y[..., D // 2:] ** 2
    assert np.max(np.abs(ny - nx) / np.maximum(nx, 1e-30)) < 4e-7


def check_bwd_after_fwd_is_identity(o):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((200, 3, 16)).astype(np.float32)
    cu = [0, 50, 51, 200]
    y = o.rope(x, cu, 1e4, 1)
    z = o.rope(y, cu, 1e4, -1)
    assert np.max(np.abs(z - x)) <= 4 * 2.0 ** -24 * np.max(np.abs(x)) * 4


def check_adjoint(o):
    """<fwd(x), g> = <x, bwd(g)>: the backward map is the transpose of the forward map."""
    rng = np.random.default_rng(16)
    cu = [0, 7, 40, 41, 90]
    x = rng.standard_normal((90, 2, 24)).astype(np.float32)
    g = rng.standard_normal((90, 2, 24)).astype(np.float32)
    lhs = np.sum(o.rope(x, cu, 1e6, 1).astype(np.float64) * g.astype(np.float64))
    rhs = np.sum(x.astype(np.float64) * o.rope(g, cu, 1e6, -1).astype(np.float64))
    scale = np.sum(np.abs(x.astype(np.float64)) * np.abs(g.astype(np.float64)))
    assert abs(lhs - rhs) < 1e-6 * scale, (lhs, rhs)


def check_packed_equals_unpacked(o):
    rng = np.random.default_rng(17)
    lengths = [3, 0, 17, 1, 40, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    for dtype in ("f32", "bf16"):
        x = (rng.standard_normal((T, 4, 16)).astype(np.float32) if dtype == "f32"
             else random_bf16(rng, (T, 4, 16)))
        packed = o.rope(x, cu, 1e6, 1, dtype)
        for s, n in enumerate(lengths):
            if n == 0:
                continue
            alone = o.rope(np.ascontiguousarray(x[cu[s]:cu[s + 1]]), [0, n], 1e6, 1, dtype)
            assert np.array_equal(packed[cu[s]:cu[s + 1]].view(np.uint32), alone.view(np.uint32))


def check_positions_golden(o):
    with open(os.path.join(GOLDEN, "positions_tiny_packed.txt")) as fh:
        lines = [ln.split() for ln in fh if ln[0] in "ps"]
    ref = {ln[0]: np.array([int(v) for v in ln[1:]], dtype=np.int32) for ln in lines}
    pos, seq = o.positions([0, 5, 22, 25, 64], 64)
    assert np.array_equal(pos, ref["pos"]) and np.array_equal(seq, ref["seq"])


def check_positions_edges(o):
    # cu[0] > 0 (tokens 0, 1 untouched), an empty sequence, seqused cutting sequence 1
    # to 2 tokens (token 4 untouched), seqused larger than its sequence, tail tokens
    # 9, 10 after cu[num_seqs] untouched. Written out by hand.
    pos, seq = o.positions([2, 2, 5, 9], 11, seqused=[0, 2, 9])
    assert pos.tolist() == [-1, -1, 0, 1, -1, 0, 1, 2, 3, -1, -1], pos
    assert seq.tolist() == [-1, -1, 1, 1, -1, 2, 2, 2, 2, -1, -1], seq
    pos, seq = o.positions([0, 0, 0], 3)
    assert pos.tolist() == [-1, -1, -1] and seq.tolist() == [-1, -1, -1]


def check_untouched_rows(o):
    rng = np.random.default_rng(18)
    x = rng.standard_normal((11, 2, 8)).astype(np.float32)
    y = o.rope(x, [2, 2, 5, 9], 1e4, 1, seqused=[0, 2, 9])
    for t in (0, 1, 4, 9, 10):
        assert np.array_equal(y[t], x[t])
    # Touched rows equal the sequence processed alone, truncated to its used length.
    alone = o.rope(np.ascontiguousarray(x[2:4]), [0, 2], 1e4, 1)
    assert np.array_equal(y[2:4], alone)
    assert not np.array_equal(y[3], x[3])


def check_exact_rounding(o):
    """The result is the exact x1*cos - x2*sin, rounded once (checked with rationals),
    also where the two products nearly cancel."""
    D, T = 8, 40
    pos = np.arange(T)
    c_half, s_half = o.cos_sin(pos, D, 1e4)
    rng = np.random.default_rng(19)
    x = np.empty((T, 1, D), dtype=np.float32)
    x[..., : D // 2] = rng.standard_normal((T, 1, D // 2)).astype(np.float32)
    # Second half chosen so that x2*sin ~= x1*cos: heavy cancellation in y1.
    with np.errstate(divide="ignore", invalid="ignore"):
        x2 = np.where(s_half[:, None, :] != 0,
                      x[..., : D // 2] * c_half[:, None, :] / s_half[:, None, :], 1.0)
    x[..., D // 2:] = x2.astype(np.float32)
    y = o.rope(x, [0, T], 1e4, 1)
    for t in range(T):
        for j in range(D // 2):
            x1, x2 = Fraction(float(x[t, 0, j])), Fraction(float(x[t, 0, j + D // 2]))
            c, s = Fraction(float(c_half[t, j])), Fraction(float(s_half[t, j]))
            assert y[t, 0, j] == rn_f32(x1 * c - x2 * s), (t, j)
            assert y[t, 0, j + D // 2] == rn_f32(x2 * c + x1 * s), (t, j)


def check_rows_match_full(o):
    rng = np.random.default_rng(20)
    cu = np.array([1, 6, 6, 30, 33], dtype=np.int32)
    su = np.array([5, 0, 20, 3], dtype=np.int32)
    T = 36
    x = random_bf16(rng, (T, 3, 16))
    full = o.rope(x, cu, 1e6, -1, "bf16", seqused=su)
    tokens = np.array([0, 35, 5, 6, 25, 26, 29, 30, 32, 33, 1, 17])
    rows = o.rope_rows(np.ascontiguousarray(x[tokens]), tokens, cu, 1e6, -1, "bf16", seqused=su)
    assert np.array_equal(rows.view(np.uint32), full[tokens].view(np.uint32))


def f16_word_value(w: int):
    """The value of a binary16 word from the IEEE 754 field layout, written in the
    textbook form: (-1)^sign * (1 + m/2^10) * 2^(e - 15) for normal words,
    (-1)^sign * (m/2^10) * 2^-14 for subnormal ones; e = 31 is an infinity (m = 0)
    or a NaN. Returns (sign, Fraction magnitude) or (sign, "inf") / (sign, "nan")."""
    sign, e, m = w >> 15, (w >> 10) & 0x1F, w & 0x3FF
    if e == 0x1F:
        return sign, ("nan" if m else "inf")
    if e == 0:
        return sign, Fraction(m, 2 ** 10) * Fraction(1, 2 ** 14)
    mag = (1 + Fraction(m, 2 ** 10))
    return sign, mag * (Fraction(2) ** (e - 15))


def check_f16_decode_all_words(o):
    """Every binary16 word (all 65536, NaNs, infinities, subnormals and -0 included)
    goes through the oracle's f16 storage path at position 0, where the rotation is
    the identity: word w in the first half of a D = 2 row (second half +0) must come
    out as the value its IEEE 754 fields define, and the same in the second half.
    Checked against the field formula above (exact rationals) and numpy's own
    binary16 widening. (In the second half the identity is x2*1 + (+0)*0, which
    turns -0 into +0 under IEEE addition; there only the zero's sign is free.)"""
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    np_vals = words.view(np.float16).astype(np.float32)
    ids = np.zeros(words.size, dtype=np.int32)  # every token at position 0
    for half in (0, 1):
        x = np.zeros((words.size, 1, 2), dtype=np.uint16)
        x[:, 0, half] = words
        y = o.rope(x, None, 1e4, 1, "f16", position_ids=ids)[:, 0, half]
        assert np.array_equal(np.isnan(y), np.isnan(np_vals)), half
        ok = ~np.isnan(y) & ((y != 0) | (half == 0))
        assert np.array_equal(y[ok].view(np.uint32), np_vals[ok].view(np.uint32)), half
        for w in range(65536):
            sign, mag = f16_word_value(w)
            v = float(y[w])
            if mag == "nan":
                assert math.isnan(v), hex(w)
                continue
            if not (half == 1 and mag == 0):
                assert math.copysign(1.0, v) == (-1.0 if sign else 1.0), hex(w)
            if mag == "inf":
                assert math.isinf(v), hex(w)
            else:
                assert Fraction(abs(v)) == mag, (hex(w), v, mag)


def check_round_bf16(o):
    import torch
    rng = np.random.default_rng(21)
    v = np.concatenate([
        rng.standard_normal(5000).astype(np.float32),
        # exact ties: 1 + 2^-8 (tie, even is 1.0), 1 + 3*2^-8 (tie, even is 1 + 2^-6),
        # and a value just above a tie
        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8),
                  0.0, -0.0, 3.0e38], dtype=np.float32),
    ])
    got = o.round_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------- NEXT rows:
# explicit position ids, per-sequence offsets, linear position interpolation.

def check_position_ids_match_cu_positions(o):
    """Explicit ids equal to the hand-written per-sample positions (golden fixture)
    give the cu_seqlens result bit for bit; negative ids leave their token alone."""
    with open(os.path.join(GOLDEN, "positions_tiny_packed.txt")) as fh:
        pos = [ln.split() for ln in fh if ln.startswith("pos")][0]
    ids = np.array([int(v) for v in pos[1:]], dtype=np.int32)
    rng = np.random.default_rng(30)
    x = random_bf16(rng, (64, 3, 16))
    for direction in (1, -1):
        a = o.rope(x, [0, 5, 22, 25, 64], 1e6, direction, "bf16")
        b = o.rope(x, None, 1e6, direction, "bf16", position_ids=ids)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ids2 = ids.copy()
    ids2[[3, 40, 63]] = -1
    b = o.rope(x, None, 1e6, 1, "bf16", position_ids=ids2)
    xf = bf16_bits_to_f32(x)
    for t in (3, 40, 63):
        assert np.array_equal(b[t].view(np.uint32), xf[t].view(np.uint32))
    pos_out, seq_out = o.positions(None, 64, position_ids=ids2)
    assert pos_out.tolist() == [(-1 if t in (3, 40, 63) else int(ids[t])) for t in range(64)]
    assert np.all(seq_out == -1)


def check_position_ids_hand_values(o):
    # D = 4, theta = 1e4: e0 with id 1 -> [cos 1, 0, sin 1, 0]; e1 with id 100 -> the
    # fp32 angle 100 * 0.01f is exactly 1 -> [0, cos 1, 0, sin 1].
    x = np.zeros((2, 1, 4), dtype=np.float32)
    x[0, 0, 0] = 1.0
    x[1, 0, 1] = 1.0
    y = o.rope(x, None, 1e4, 1, position_ids=[1, 100])
    c1, s1 = np.float32(math.cos(1.0)), np.float32(math.sin(1.0))
    assert y[0, 0].tolist() == [c1, 0.0, s1, 0.0] and y[1, 0].tolist() == [0.0, c1, 0.0, s1], y


def check_seq_offsets_shard_invariant(o):
    """A long sequence cut into shards, each rotated with the global position of its
    first token as offset, gives exactly the unsharded result (sequence/context
    parallelism needs nothing else from RoPE)."""
    rng = np.random.default_rng(31)
    L = 97
    x = random_bf16(rng, (L, 2, 32))
    full = o.rope(x, [0, L], 1e6, 1, "bf16")
    cuts = [0, 20, 21, 60, L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = o.rope(np.ascontiguousarray(x[a:b]), [0, b - a], 1e6, 1, "bf16", seq_offsets=[a])
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)
    # Two packed shards of two different sequences in one call.
    both = np.concatenate([x[20:60], x[60:L]])
    y = o.rope(both, [0, 40, 40 + L - 60], 1e6, 1, "bf16", seq_offsets=[20, 60])
    assert np.array_equal(y.view(np.uint32), full[20:L].view(np.uint32))
    # A negative shifted position leaves its token untouched.
    pos, seq = o.positions([0, 4], 4, seq_offsets=[-2])
    assert pos.tolist() == [-1, -1, 0, 1] and seq.tolist() == [-1, -1, 0, 0]


def check_pos_scale_page_example(o):
    """With factor 4, position 100000 is treated as position 25000 (TRL guide, YaRN
    section): same cos/sin bit for bit, and the scaled rotation of positions 4p
    equals the unscaled rotation of positions p."""
    c4, s4 = o.cos_sin([100000], 128, 1e6, pos_scale=4.0)
    c1, s1 = o.cos_sin([25000], 128, 1e6)
    assert np.array_equal(c4.view(np.uint32), c1.view(np.uint32))
    assert np.array_equal(s4.view(np.uint32), s1.view(np.uint32))
    rng = np.random.default_rng(32)
    x = random_bf16(rng, (50, 2, 16))
    p = np.arange(50, dtype=np.int32) * 37
    a = o.rope(x, None, 1e4, 1, "bf16", position_ids=4 * p, pos_scale=4.0)
    b = o.rope(x, None, 1e4, 1, "bf16", position_ids=p)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def check_pos_scale_mpmath(o):
    """Scaled angle = fp32(fp32(pos) / fp32(factor)) * inv_freq, one rounding per step;
    cos/sin correctly rounded (mpmath)."""
    D, theta = 64, 5e5
    f = ref_inv_freq(theta, D)
    plist = [1, 3, 7, 999, 40961, 163839, 524287]
    for factor in (1.5, 2.5, 4.0):
        c, s = o.cos_sin(plist, D, theta, pos_scale=factor)
        for i, p in enumerate(plist):
            sp = np.float32(np.float32(p) / np.float32(factor))
            for j in range(D // 2):
                a = mpmath.mpf(float(np.float32(sp * f[j])))
                assert c[i, j] == rn_f32(mpmath.cos(a)), (factor, p, j)
                assert s[i, j] == rn_f32(mpmath.sin(a)), (factor, p, j)


# ------------------------------------------------------- caller-supplied cos/sin tables

def check_table_block_matrix_R(o):
    """With arbitrary tables (not cos/sin of anything, not on the unit circle), the
    table rotation is x*C + (x @ R)*S with R, R^T from the page's block form, each
    token using the table row of its position; positions without a row, and tokens
    outside every sequence, are untouched."""
    mats = load_golden_matrices()
    rng = np.random.default_rng(31)
    for D in (4, 6):
        R, RT = mats[("R", D)], mats[("RT", D)]
        T, H, rows = 14, 2, 5
        x = rng.standard_normal((T, H, D)).astype(np.float32)
        cu = np.array([1, 4, 12], dtype=np.int32)   # token 0 and 12, 13 outside
        pos = [-1, 0, 1, 2, 0, 1, 2, 3, 4, 5, 6, 7, -1, -1]  # rows 5.. do not exist
        ct = rng.uniform(-1.5, 1.5, (rows, D // 2)).astype(np.float32)
        st = rng.uniform(-1.5, 1.5, (rows, D // 2)).astype(np.float32)
        xd = x.astype(np.float64)
        for direction, M in ((1, R), (-1, RT)):
            got = o.rope_table(x, cu, ct, st, direction)
            for t in range(T):
                p = pos[t]
                if p < 0 or p >= rows:
                    assert np.array_equal(got[t].view(np.uint32), x[t].view(np.uint32)), t
                    continue
                C, S = full_cos_sin(ct[p:p + 1].astype(np.float64), st[p:p + 1].astype(np.float64))
                # rotate_half's sign lives in R / R^T: S stays the table's sin both ways
                ref = (xd[t] * C[0] + (xd[t] @ M) * S[0]).astype(np.float32)
                assert np.array_equal(got[t].view(np.uint32), ref.view(np.uint32)), (D, direction, t)


def check_table_equals_theta(o):
    """Tables holding the oracle's own cos/sin of positions 0..rows-1 reproduce the
    theta path bit for bit (packed with seqused, per-sequence offsets, explicit ids)."""
    rng = np.random.default_rng(32)
    D, H, theta = 16, 3, 1e6
    cu = np.array([0, 5, 5, 17, 30], dtype=np.int32)
    su = np.array([4, 0, 12, 9], dtype=np.int32)
    so = np.array([3, 0, 100, 7], dtype=np.int32)
    T = 32
    pid = rng.integers(-2, 120, T).astype(np.int32)
    rows = 130
    ct, st = o.cos_sin(np.arange(rows), D, theta)
    x = random_bf16(rng, (T, H, D))
    for direction in (1, -1):
        for kw in (dict(seqused=su), dict(seq_offsets=so), dict(position_ids=pid)):
            ref = o.rope(x, cu, theta, direction, "bf16", **kw)
            got = o.rope_table(x, cu, ct, st, direction, "bf16", **kw)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (direction, kw)


def check_table_hand_values(o):
    """cos = 1, sin = 0 is the identity; cos = 0, sin = 1 is rotate_half exactly:
    forward [x1, x2] -> [-x2, x1], backward -> [x2, -x1]."""
    rng = np.random.default_rng(33)
    D, T = 8, 3
    x = rng.standard_normal((T, 1, D)).astype(np.float32)
    one, zero = np.ones((1, D // 2), np.float32), np.zeros((1, D // 2), np.float32)
    cu = [0, T]
    pid = np.zeros(T, dtype=np.int32)
    ident = o.rope_table(x, cu, one, zero, 1, position_ids=pid)
    assert np.array_equal(ident, x)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    fwd = o.rope_table(x, cu, zero, one, 1, position_ids=pid)
    bwd = o.rope_table(x, cu, zero, one, -1, position_ids=pid)
    assert np.array_equal(fwd, np.concatenate([-x2, x1], axis=-1))
    assert np.array_equal(bwd, np.concatenate([x2, -x1], axis=-1))


ALL_CHECKS = [
    check_inv_freq_closed_form,
    check_inv_freq_mpmath,
    check_cos_sin_pos0,
    check_cos_sin_mpmath,
    check_block_matrix_R,
    check_complex_form,
    check_hand_values,
    check_identity_at_pos0,
    check_pair_norm,
    check_bwd_after_fwd_is_identity,
    check_adjoint,
    check_packed_equals_unpacked,
    check_positions_golden,
    check_positions_edges,
    check_untouched_rows,
    check_exact_rounding,
    check_rows_match_full,
    check_round_bf16,
    check_f16_decode_all_words,
    check_position_ids_match_cu_positions,
    check_position_ids_hand_values,
    check_seq_offsets_shard_invariant,
    check_pos_scale_page_example,
    check_pos_scale_mpmath,
    check_table_block_matrix_R,
    check_table_equals_theta,
    check_table_hand_values,
]
