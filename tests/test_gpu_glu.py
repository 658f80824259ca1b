"""GPU parity of the SwiGLU / GeGLU kernels (called through the C ABI via the
Python binding) against the CPU oracle on the same seeded inputs.

Bars (derived from the fp32 arithmetic of the kernels, written here):
  * bf16 / f16 storage: every output within 1 ulp of the oracle's double result
    rounded once to the storage dtype (ordered-bit distance, +0 == -0). The
    kernels' fp32 results are within a few fp32 ulps of the exact value (the
    derivative's root is handled by a Taylor polynomial), far below half a 16-bit
    ulp, so only the final rounding can differ.
  * f32 storage: |gpu - ref| <= (16 + B tail(e)) fp32 ulps of the exact value,
    where tail(e) is the conditioning of the kind's tail in fp32 arithmetic
    (SwiGLU: none, B = 0; exact GeGLU: e^2 from the erfc tail, B = 2; tanh GeGLU:
    |2u(e)|, the rounding of the fp32 argument of exp(2u) amplified in its tail,
    B = 12). Measured worst cases on 4M elements with e ~ N(0, 16): SwiGLU 9.6 ulps,
    exact GeGLU 11.5 + 1.31 e^2, tanh GeGLU 8.8 + 7.13 |2u|
    (test_glu_f32_accuracy prints them). Where the exponential inside falls below
    the fp32 normal range (|e| > 87 for SwiGLU, |e| > 13 for the exact GELU, |2u| >
    87 for the tanh form) it keeps only its subnormal steps of 2^-149, so an
    absolute allowance of 16 such steps times the factors that multiply it (|g|,
    |dh g| or |dh|, times 1 + |e|, and 1 + e^2 more for the tanh form's de) is
    added; it is below 2^-120 wherever the inputs are of order one.
  * layout variants (access width, dense vs strided, 32- vs 64-bit offsets,
    in place): bit-identical to each other.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import glu as glu_oracle

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))
DEV = torch.device("cuda:0")
KINDS = ("swiglu", "geglu", "geglu_tanh")
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def rope():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_rotary_rope_amd as m
    return m


def words(t: torch.Tensor) -> np.ndarray:
    """Storage of a tensor (any strides) as numpy: float32 values or uint16 words."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def values(w: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return w.astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(TORCH_DT[dtype])
    return t.double().numpy()


def ordered16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


F32_ULPS = {"swiglu": (16.0, 0.0), "geglu": (16.0, 2.0), "geglu_tanh": (16.0, 12.0)}


def assert_glu_parity(dtype: str, got: np.ndarray, ref: np.ndarray, e_vals: np.ndarray, what: str,
                      kind: str | None = None, underflow_scale=None):
    got = got.reshape(ref.shape)
    if dtype == "f32":
        g = got.astype(np.float64)
        a, b = F32_ULPS[kind]
        ok = f32_ulps(g, ref) <= a + b * f32_tail(kind, e_vals)
        if underflow_scale is not None:
            ok |= np.abs(g - ref) <= 16 * 2.0 ** -149 * underflow_scale
        # where the exact result overflows fp32, the correctly rounded answer is +-inf
        over = np.isinf(glu_oracle.round_to("f32", ref))
        ok[over] = g[over] == glu_oracle.round_to("f32", ref)[over]
        bad = ~ok
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of bound, first at "
                               f"e={e_vals[bad][0]!r} got={g[bad][0]!r} ref={ref[bad][0]!r}")
    else:
        want = glu_oracle.round_to(dtype, ref)
        d = np.abs(ordered16(got) - ordered16(want))
        bad = d > 1
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1 ulp (worst "
                               f"{int(d.max())}), first at e={e_vals[bad][0]!r} "
                               f"got={got[bad][0]:#06x} want={want[bad][0]:#06x}")


def make(shape, seed, dtype, scale=1.0):
    t = workloads.make_tensor(shape, seed, dtype, device=DEV, chunk_rows=4096)
    return t if scale == 1.0 else (t.float() * scale).to(TORCH_DT[dtype])


def check_all(rope, kind, dtype, e, g, dh, what):
    """Run fwd and bwd on the given GPU tensors and compare with the oracle."""
    h = rope.glu_fwd(kind, e, g)
    de, dg = rope.glu_bwd(kind, dh, e, g)
    torch.cuda.synchronize()
    we, wg, wd = words(e), words(g), words(dh)
    ev = values(we, dtype)
    ref_h = glu_oracle.fwd(kind, we, wg, dtype, NTHREADS)
    ref_de, ref_dg = glu_oracle.bwd(kind, wd, we, wg, dtype, NTHREADS)
    gv, dv = np.abs(values(wg, dtype)), np.abs(values(wd, dtype))
    grow = 1.0 + np.abs(ev)
    scale = {"h": gv * grow, "de": dv * gv * grow * (1.0 + ev * ev if kind == "geglu_tanh" else 1.0),
             "dg": dv * grow}
    assert_glu_parity(dtype, words(h), ref_h, ev, f"{what}:{kind}:h", kind, scale["h"])
    assert_glu_parity(dtype, words(de), ref_de, ev, f"{what}:{kind}:de", kind, scale["de"])
    assert_glu_parity(dtype, words(dg), ref_dg, ev, f"{what}:{kind}:dg", kind, scale["dg"])
    return h, de, dg


# ---------------------------------------------------------------- whole workloads

@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("name", ["glu_tiny", "glu_qwen3_8b", "glu_qwen3_4b"])
def test_glu_workload_parity(rope, name, kind):
    w = workloads.glu_get(name)
    print(f"[glu parity] {name} {kind}", flush=True)
    e = make((w.rows, w.cols), w.seed("e"), w.dtype)
    g = make((w.rows, w.cols), w.seed("g"), w.dtype)
    dh = make((w.rows, w.cols), w.seed("dh"), w.dtype)
    check_all(rope, kind, w.dtype, e, g, dh, name)


def f32_tail(kind: str, e: np.ndarray) -> np.ndarray:
    """The conditioning of each kind's tail for fp32 arithmetic: e^2 for the exact
    GELU's erfc tail, |2u(e)| = |2 sqrt(2/pi) (e + 0.044715 e^3)| for the tanh form's
    exp(2u) tail, none for SwiGLU."""
    if kind == "geglu":
        return e * e
    if kind == "geglu_tanh":
        return np.abs(2 * math.sqrt(2 / math.pi) * (e + 0.044715 * e ** 3))
    return np.zeros_like(e)


def f32_ulps(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """|got - ref| in units of the fp32 ulp at the exact value ref (normal range;
    below it the smallest subnormal step)."""
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(mag)) - 23)
    return np.abs(got.astype(np.float64) - ref) / ulp


@pytest.mark.parametrize("kind", KINDS)
def test_glu_f32_accuracy(rope, kind):
    """fp32 storage on 4096 x 1024 elements, e ~ N(0, 4^2) (so the tails out to
    |e| ~ 20 are sampled), against the oracle; reports the worst error in fp32 ulps
    per |e| band for each output."""
    rows, cols = 4096, 1024
    print(f"[glu f32 accuracy] {kind}", flush=True)
    e = make((rows, cols), 9900, "f32", scale=4.0)
    g = make((rows, cols), 9901, "f32")
    dh = make((rows, cols), 9902, "f32")
    h, de, dg = check_all(rope, kind, "f32", e, g, dh, "f32acc")
    we, wg, wd = words(e), words(g), words(dh)
    ref = {"h": glu_oracle.fwd(kind, we, wg, "f32", NTHREADS)}
    ref["de"], ref["dg"] = glu_oracle.bwd(kind, wd, we, wg, "f32", NTHREADS)
    ev = we.astype(np.float64)
    ae = np.abs(ev)
    tail = f32_tail(kind, ev)
    bands = [(0, 1), (1, 2), (2, 4), (4, 8), (8, 16), (16, 1e9)]
    for name, got in (("h", h), ("de", de), ("dg", dg)):
        u = f32_ulps(words(got), ref[name])
        worst = [float(u[(ae >= a) & (ae < b)].max()) if ((ae >= a) & (ae < b)).any() else 0.0
                 for a, b in bands]
        A = float(u[ae < 2].max())
        big = (ae >= 2) & (tail > 0)
        B = float((u[big] / tail[big]).max()) if big.any() else 0.0
        print(f"[glu f32 ulps] {kind} {name}: A={A:.1f} B={B:.3f} " +
              " ".join(f"|e|in[{a},{b}):{w:.1f}" for (a, b), w in zip(bands, worst)), flush=True)


# ---------------------------------------------------------------- edge values

def edge_values(dtype: str) -> np.ndarray:
    """Zeros, tiny and subnormal magnitudes, the neighbourhoods of the derivative
    roots (every representable value nearby for 16-bit types, ulp steps for f32),
    the exp/erfc underflow region and huge magnitudes."""
    ft = TORCH_DT[dtype]
    info = torch.finfo(ft)
    base = [0.0, -0.0, 1e-30, -1e-30, 1e-39, -1e-39, 1e-41, -3e-42, info.tiny, -info.tiny,
            0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0, 5.0, -5.0, 8.0, -8.0, 10.0, -10.0,
            12.5, -12.5, 13.5, -13.5, 20.0, -20.0, 40.0, -40.0, 64.0, -64.0, 65.0, -65.0,
            87.0, -87.0, 88.5, -88.5, 90.0, -90.0, 95.0, -95.0, 100.0, -100.0, 104.0, -104.0,
            110.0, -110.0, 1e4, -1e4, info.max, -info.max]
    vals = torch.tensor(base, dtype=torch.float64).to(ft)
    roots = [-1.2784645427610738, -0.7517915246935645, -0.7524614220710163]
    steps = []
    for r in roots:
        c = torch.tensor([r], dtype=torch.float64).to(ft)
        x = c.clone()
        for _ in range(40):  # 40 representable values each side
            x = torch.nextafter(x, torch.tensor([-np.inf], dtype=ft))
            steps.append(x.clone())
        x = c.clone()
        for _ in range(40):
            x = torch.nextafter(x, torch.tensor([np.inf], dtype=ft))
            steps.append(x.clone())
        steps.append(c)
        # the window edges of the Taylor polynomial and just beyond
        for d in (0.2499, 0.25, 0.2501, 0.3):
            steps.append(torch.tensor([r - d, r + d], dtype=torch.float64).to(ft))
    vals = torch.cat([vals] + steps)
    return vals.float().numpy() if dtype == "f32" else words(vals)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_glu_edge_values(rope, kind, dtype):
    print(f"[glu parity] edge values {kind} {dtype}", flush=True)
    ev = edge_values(dtype)
    n = ev.size
    ft = TORCH_DT[dtype]
    if dtype == "f32":
        e = torch.from_numpy(ev).to(DEV).view(1, n)
    else:
        e = torch.from_numpy(ev.view(np.int16)).view(ft).to(DEV).view(1, n)
    rng = np.random.default_rng(21)
    g = torch.from_numpy(rng.standard_normal((1, n)).astype(np.float32)).to(ft).to(DEV)
    dh = torch.from_numpy(rng.standard_normal((1, n)).astype(np.float32)).to(ft).to(DEV)
    check_all(rope, kind, dtype, e, g, dh, f"edge:{dtype}")


# ---------------------------------------------------------------- layouts

@pytest.mark.parametrize("kind", KINDS)
def test_fused_gate_up_layout(rope, kind):
    """e and g as the two halves of one fused gate/up output [rows, 2*cols] (row
    stride 2*cols): bit-identical to dense copies, gradients land in a fused
    buffer, and the oracle agrees."""
    rows, cols = 1000, 1536
    print(f"[glu parity] fused gate/up {kind}", flush=True)
    gu = make((rows, 2 * cols), 9400, "bf16")
    dh = make((rows, cols), 9401, "bf16")
    e, g = gu[:, :cols], gu[:, cols:]
    h = rope.glu_fwd(kind, e, g)
    de, dg = rope.glu_bwd(kind, dh, e, g)
    assert de.stride(0) == 2 * cols and dg.data_ptr() == de.data_ptr() + cols * 2
    h2 = rope.glu_fwd(kind, e.contiguous(), g.contiguous())
    de2, dg2 = rope.glu_bwd(kind, dh, e.contiguous(), g.contiguous())
    torch.cuda.synchronize()
    for a, b in ((h, h2), (de, de2), (dg, dg2)):
        assert np.array_equal(words(a), words(b))
    we, wg = words(e), words(g)
    ref_h = glu_oracle.fwd(kind, we, wg, "bf16", NTHREADS)
    assert_glu_parity("bf16", words(h), ref_h, values(we, "bf16"), f"fused:{kind}:h")


@pytest.mark.parametrize("kind", KINDS)
def test_split_call_fused_layout(rope, kind):
    """A call long enough to go out as several launches on the 32-bit path: 70001 rows
    x 7680 bf16 as the halves of a fused gate/up output (65626 workgroups of 1024
    16-byte chunks: 3 launches of 21880, 21880 and 21866 workgroups, whose boundaries
    fall inside rows 23338 and 46677). Bit-identical to dense copies of e and g;
    rows around the launch boundaries and every 37th row against the oracle,
    forward and backward."""
    rows, cols = 70001, 7680
    print(f"[glu parity] split call, fused gate/up {kind}", flush=True)
    gu = make((rows, 2 * cols), 9450, "bf16")
    dh = make((rows, cols), 9451, "bf16")
    e, g = gu[:, :cols], gu[:, cols:]
    h = rope.glu_fwd(kind, e, g)
    de, dg = rope.glu_bwd(kind, dh, e, g)
    ec, gc = e.contiguous(), g.contiguous()
    h2 = rope.glu_fwd(kind, ec, gc)
    de2, dg2 = rope.glu_bwd(kind, dh, ec, gc)
    torch.cuda.synchronize()
    for a, b in ((h, h2), (de, de2), (dg, dg2)):
        assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    chunks_per_row = cols // 8
    edges = [21880 * 1024 * m // chunks_per_row for m in (1, 2)]
    assert edges == [23338, 46677]
    sel = np.unique(np.concatenate([np.arange(0, 3), np.arange(rows - 3, rows),
                                    *[np.arange(r - 2, r + 3) for r in edges],
                                    np.arange(0, rows, 37)]))
    idx = torch.from_numpy(sel).to(DEV)
    we, wg, wd = (words(t.index_select(0, idx)) for t in (e, g, dh))
    ev = values(we, "bf16")
    ref_h = glu_oracle.fwd(kind, we, wg, "bf16", NTHREADS)
    ref_de, ref_dg = glu_oracle.bwd(kind, wd, we, wg, "bf16", NTHREADS)
    assert_glu_parity("bf16", words(h.index_select(0, idx)), ref_h, ev, f"split:{kind}:h")
    assert_glu_parity("bf16", words(de.index_select(0, idx)), ref_de, ev, f"split:{kind}:de")
    assert_glu_parity("bf16", words(dg.index_select(0, idx)), ref_dg, ev, f"split:{kind}:dg")
    del gu, dh, e, g, h, de, dg, ec, gc, h2, de2, dg2
    torch.cuda.empty_cache()


def test_split_call_f32(rope):
    """fp32 storage, a call of 65544 workgroups on the 32-bit path (8193 rows x 32768,
    4-element chunks: 3 launches of 21848 workgroups): rows around
    the launch boundaries and every 41st row against the oracle, forward and
    backward, within the fp32 bound."""
    rows, cols = 8193, 32768
    print("[glu parity] split call f32", flush=True)
    e = make((rows, cols), 9460, "f32")
    g = make((rows, cols), 9461, "f32")
    dh = make((rows, cols), 9462, "f32")
    h = rope.glu_fwd("swiglu", e, g)
    de, dg = rope.glu_bwd("swiglu", dh, e, g)
    torch.cuda.synchronize()
    chunks_per_row = cols // 4
    edges = [21848 * 1024 * m // chunks_per_row for m in (1, 2)]
    sel = np.unique(np.concatenate([np.arange(0, 2), np.arange(rows - 2, rows),
                                    *[np.arange(r - 1, r + 2) for r in edges],
                                    np.arange(0, rows, 41)]))
    idx = torch.from_numpy(sel).to(DEV)
    we, wg, wd = (words(t.index_select(0, idx)) for t in (e, g, dh))
    ev = values(we, "f32")
    ref_h = glu_oracle.fwd("swiglu", we, wg, "f32", NTHREADS)
    ref_de, ref_dg = glu_oracle.bwd("swiglu", wd, we, wg, "f32", NTHREADS)
    gv, dv = np.abs(values(wg, "f32")), np.abs(values(wd, "f32"))
    grow = 1.0 + np.abs(ev)
    assert_glu_parity("f32", words(h.index_select(0, idx)), ref_h, ev, "split-f32:h", "swiglu",
                      gv * grow)
    assert_glu_parity("f32", words(de.index_select(0, idx)), ref_de, ev, "split-f32:de", "swiglu",
                      dv * gv * grow)
    assert_glu_parity("f32", words(dg.index_select(0, idx)), ref_dg, ev, "split-f32:dg", "swiglu",
                      dv * grow)
    del e, g, dh, h, de, dg
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,cols,lead,in_pad,out_pad", [
    ("bf16", 1000, 0, 0, 0),     # 16-byte chunks, dense
    ("bf16", 1000, 4, 0, 0),     # base 8 bytes off: 8-byte chunks
    ("bf16", 998, 2, 0, 0),      # 4-byte chunks
    ("bf16", 999, 1, 0, 0),      # odd row length: 2-byte chunks
    ("bf16", 1000, 0, 8, 24),    # strided rows, 16-byte chunks
    ("f16", 1001, 0, 3, 5),      # strided, odd
    ("f32", 1000, 0, 0, 0),
    ("f32", 1002, 2, 2, 0),      # 8-byte chunks, strided
    ("f32", 1001, 1, 0, 0),      # 4-byte chunks
])
def test_layout_variants_bit_identical(rope, dtype, cols, lead, in_pad, out_pad):
    """Access widths, strides and forced 32- or 64-bit offsets all give the dense
    default's bits; gap elements are never written."""
    rows = 257
    ft = TORCH_DT[dtype]
    print(f"[glu parity] layouts {dtype} cols={cols} lead={lead} pads={in_pad},{out_pad}",
          flush=True)
    e0 = make((rows, cols), 9500 + cols, dtype, scale=2.0)
    g0 = make((rows, cols), 9600 + cols, dtype)
    d0 = make((rows, cols), 9700 + cols, dtype)
    ref = {}
    for kind in KINDS:
        h = rope.glu_fwd(kind, e0, g0)
        de, dg = rope.glu_bwd(kind, d0, e0, g0)
        ref[kind] = (h, de, dg)
    istride, ostride = cols + in_pad, cols + out_pad
    ebuf = torch.full((rows * istride + lead,), float("nan"), dtype=ft, device=DEV)
    gbuf = torch.full_like(ebuf, float("nan"))
    dbuf = torch.full((rows * ostride + lead,), float("nan"), dtype=ft, device=DEV)
    hbuf = torch.full_like(dbuf, 7.0)
    e = ebuf[lead:].as_strided((rows, cols), (istride, 1))
    g = gbuf[lead:].as_strided((rows, cols), (istride, 1))
    dh = dbuf[lead:].as_strided((rows, cols), (ostride, 1))
    hv = hbuf[lead:].as_strided((rows, cols), (ostride, 1))
    e.copy_(e0)
    g.copy_(g0)
    dh.copy_(d0)
    for kind in KINDS:
        for mode in (rope.INDEX_AUTO, rope.INDEX_32, rope.INDEX_64):
            rope.glu_fwd(kind, e, g, out=hv, index_mode=mode)
            de, dg = rope.glu_bwd(kind, dh, e, g, index_mode=mode)
            torch.cuda.synchronize()
            for a, b in zip((hv, de, dg), ref[kind]):
                assert np.array_equal(words(a), words(b)), (kind, mode)
    untouched = torch.ones(rows * ostride + lead, dtype=torch.bool, device=DEV)
    untouched[lead:].view(-1)[:rows * ostride].view(rows, ostride)[:, :cols] = False
    assert bool((hbuf[untouched] == 7.0).all())


@pytest.mark.parametrize("kind", KINDS)
def test_in_place(rope, kind):
    """h written over e, then de over e and dg over g (fully in-place backward):
    bit-identical to the out-of-place results."""
    rows, cols = 300, 2048
    print(f"[glu parity] in place {kind}", flush=True)
    e0 = make((rows, cols), 9800, "bf16", scale=2.0)
    g0 = make((rows, cols), 9801, "bf16")
    d0 = make((rows, cols), 9802, "bf16")
    h_ref = rope.glu_fwd(kind, e0, g0)
    de_ref, dg_ref = rope.glu_bwd(kind, d0, e0, g0)
    e1 = e0.clone()
    rope.glu_fwd(kind, e1, g0, out=e1)
    e2, g2 = e0.clone(), g0.clone()
    rope.glu_bwd(kind, d0, e2, g2, de=e2, dg=g2)
    torch.cuda.synchronize()
    assert np.array_equal(words(e1), words(h_ref))
    assert np.array_equal(words(e2), words(de_ref))
    assert np.array_equal(words(g2), words(dg_ref))


def test_empty(rope):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert rope.glu_fwd("swiglu", x, x).shape == (0, 64)
    y = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    de, dg = rope.glu_bwd("geglu", y, y, y)
    assert de.shape == (5, 0)


@pytest.mark.parametrize("kind", KINDS)
def test_long_context_int64(rope, kind):
    """524288 tokens x 9728 (5.1e9 elements, 2.4 x 2^31): the 64-bit path, for each
    kind, as 19 launches of 32768 workgroups (8192 elements each). Forward and
    in-place backward; rows at the start, around the 2^31-element boundary, around
    every launch boundary, at the end, and every 97th row (a prime stride, so the
    sampled rows' offsets take every residue of the power-of-two tile sizes) against
    the oracle."""
    w = workloads.glu_get("glu_long_512k")
    print(f"[glu parity] glu_long_512k int64 path {kind}", flush=True)
    assert w.elements >= 2 ** 31
    e = workloads.make_tensor((w.rows, w.cols), w.seed("e"), w.dtype, device=DEV, chunk_rows=32768)
    g = workloads.make_tensor((w.rows, w.cols), w.seed("g"), w.dtype, device=DEV, chunk_rows=32768)
    h = rope.glu_fwd(kind, e, g)
    with pytest.raises(rope.RopeError):
        rope.glu_fwd(kind, e, g, out=h, index_mode=rope.INDEX_32)
    boundary_row = (2 ** 31) // w.cols
    launch_rows = [m * 32768 * 8192 // w.cols for m in range(1, 19)]
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(boundary_row - 2, boundary_row + 3),
                                     *[np.arange(r - 1, r + 2) for r in launch_rows],
                                     np.arange(w.rows - 4, w.rows), np.arange(0, w.rows, 97)]))
    idx = torch.from_numpy(rows).to(DEV)
    e_s, g_s = words(e.index_select(0, idx)), words(g.index_select(0, idx))
    ev = values(e_s, w.dtype)
    torch.cuda.synchronize()
    ref_h = glu_oracle.fwd(kind, e_s, g_s, w.dtype, NTHREADS)
    assert_glu_parity(w.dtype, words(h.index_select(0, idx)), ref_h, ev, f"long:{kind}:h")
    dh = h  # reuse the buffer as the upstream gradient (any values will do)
    d_s = words(dh.index_select(0, idx))
    rope.glu_bwd(kind, dh, e, g, de=e, dg=g)
    torch.cuda.synchronize()
    ref_de, ref_dg = glu_oracle.bwd(kind, d_s, e_s, g_s, w.dtype, NTHREADS)
    assert_glu_parity(w.dtype, words(e.index_select(0, idx)), ref_de, ev, f"long:{kind}:de")
    assert_glu_parity(w.dtype, words(g.index_select(0, idx)), ref_dg, ev, f"long:{kind}:dg")
    del e, g, h, dh
    torch.cuda.empty_cache()
