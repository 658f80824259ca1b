"""GPU parity: the HIP library, called through its C ABI (via the Python
binding), against the CPU oracle on the same seeded inputs.

Bars (written here, per dtype):
  * fp32 storage: max |gpu - oracle| <= 1e-5 * max|x| over each tensor;
  * bf16 / fp16 storage: every element within 1 ulp of the oracle's fp32 result
    rounded to the storage dtype (ordered-bit distance, +0 == -0);
  * positions, sequence ids and untouched rows: bit-exact;
  * cos/sin exports: bit-exact against the oracle's correctly rounded values.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))
DEV = torch.device("cuda:0")
CANARY = {"f32": 0x7FA5A5A5, "bf16": 0x7FA5, "f16": 0x7D25}  # signalling NaNs


@pytest.fixture(scope="module")
def rope():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_rotary_rope_amd as m
    return m


def bits(t: torch.Tensor) -> np.ndarray:
    return workloads.host_bits(t)


def ordered(b: np.ndarray, width: int) -> np.ndarray:
    """Map float bit patterns to integers ordered like the values (+0 and -0 -> 0)."""
    b = b.astype(np.int64)
    sign = 1 << (width - 1)
    return np.where(b & sign, -(b & (sign - 1)), b)


def round_ref(ref32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return oracle.round_bf16(ref32)
    return ref32.astype(np.float16).view(np.uint16)  # numpy: round to nearest even


def assert_parity(dtype, got, ref32, x, touched, what):
    """got, x: storage bits (float32 array for f32, uint16 words otherwise); ref32: oracle."""
    got, x, ref32 = got.reshape(got.shape[0], -1), x.reshape(x.shape[0], -1), \
        ref32.reshape(ref32.shape[0], -1)
    # untouched rows: bit-for-bit
    if (~touched).any():
        gu = got[~touched].view(np.uint32 if dtype == "f32" else np.uint16)
        xu = x[~touched].view(np.uint32 if dtype == "f32" else np.uint16)
        assert np.array_equal(gu, xu), f"{what}: an untouched row changed"
    g, r = got[touched], ref32[touched]
    if dtype == "f32":
        xmax = float(np.max(np.abs(x[touched]))) if g.size else 0.0
        err = float(np.max(np.abs(g.astype(np.float64) - r.astype(np.float64)))) if g.size else 0.0
        assert err <= 1e-5 * xmax, f"{what}: max abs err {err} > 1e-5 * {xmax}"
    else:
        want = round_ref(r, dtype)
        neq = g != want  # the ulp distance is needed only where the bits differ
        d = np.abs(ordered(g[neq], 16) - ordered(want[neq], 16))
        worst = int(d.max()) if d.size else 0
        assert worst <= 1, f"{what}: {int((d > 1).sum())} elements beyond 1 ulp (worst {worst})"


def _word(dtype: torch.dtype):
    return torch.int32 if dtype == torch.float32 else torch.int16


def _canary(dtype: torch.dtype) -> int:
    return {torch.float32: CANARY["f32"], torch.bfloat16: CANARY["bf16"],
            torch.float16: CANARY["f16"]}[dtype]


def guarded(t_host: torch.Tensor, guard: int = 4096):
    """Copy t_host to the GPU inside a larger buffer whose guard regions hold canaries.
    Returns (view on the GPU, flat buffer, guard)."""
    n = t_host.numel()
    flat = torch.empty(n + 2 * guard, dtype=t_host.dtype, device=DEV)
    flat.view(_word(t_host.dtype)).fill_(_canary(t_host.dtype))  # canaries fit the signed word
    view = flat[guard:guard + n].view(t_host.shape)
    view.copy_(t_host)
    return view, flat, guard


def guards_intact(flat: torch.Tensor, guard: int) -> bool:
    g = torch.cat([flat[:guard], flat[-guard:]]).view(_word(flat.dtype))
    return bool(torch.all(g == _canary(flat.dtype)))


def run_and_check(rope, w, host, cu_np, su_np, theta, dtype, apply_kw=None, guard=True):
    """host: dict of CPU tensors q, k, dq, dk. Runs fwd on (q, k) and bwd on (dq, dk)."""
    print(f"[parity] {w} T={host['q'].shape[0]} Hq={host['q'].shape[1]} "
          f"Hkv={host['k'].shape[1]} D={host['q'].shape[2]} {dtype} {apply_kw or ''}", flush=True)
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).to(DEV)
    su = None if su_np is None else torch.from_numpy(np.asarray(su_np, dtype=np.int32)).to(DEV)
    dev, flats = {}, {}
    for what, t in host.items():
        if guard:
            dev[what], flats[what], g = guarded(t)
        else:
            dev[what] = t.to(DEV)
    if apply_kw is None:
        rope.qk_fwd_(dev["q"], dev["k"], cu, theta, seqused=su)
        rope.qk_bwd_(dev["dq"], dev["dk"], cu, theta, seqused=su)
    else:
        rope.qk_apply_(dev["q"], dev["k"], cu, theta, 1, seqused=su, **apply_kw)
        rope.qk_apply_(dev["dq"], dev["dk"], cu, theta, -1, seqused=su, **apply_kw)
    torch.cuda.synchronize()
    T = host["q"].shape[0]
    pos, _ = oracle.positions(cu_np, T, su_np)
    touched = pos >= 0
    out = {}
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        x = bits(host[what])
        got = bits(dev[what])
        ref = oracle.rope(x, cu_np, theta, direction, dtype, su_np, NTHREADS)
        assert_parity(dtype, got, ref, x, touched, f"{w}:{what}")
        if guard:
            assert guards_intact(flats[what], g), f"{w}:{what}: guard region written"
        out[what] = got
    return out


def make_host(w: workloads.Workload, canary_untouched: bool = True):
    host = {what: workloads.make_tensor(w.shape(what), w.seed(what), w.dtype)
            for what in ("q", "k", "dq", "dk")}
    if canary_untouched:
        pos, _ = oracle.positions(w.cu_seqlens, w.T, w.seqused)
        un = torch.from_numpy(pos < 0)
        if un.any():
            for t in host.values():
                t.view(_word(t.dtype))[un] = CANARY[w.dtype]
    return host


# ---------------------------------------------------------------- full workloads

@pytest.mark.parametrize("name", ["tiny_packed", "qwen3_4b_packed", "qwen3_8b_packed",
                                  "qwen3_8b_padded", "qwen3_32b_packed"])
def test_workload_parity(rope, name):
    w = workloads.get(name)
    host = make_host(w)
    run_and_check(rope, name, host, w.cu_seqlens, w.seqused, w.theta, w.dtype)


def test_padded_equals_packed(rope):
    """The padded layout with seqused gives, row for row, the packed layout's result."""
    a, b = workloads.get("qwen3_8b_packed"), workloads.get("qwen3_8b_padded")
    print("[parity] packed vs padded qwen3_8b", flush=True)
    qa = workloads.make_tensor(a.shape("q"), 77, "bf16").to(DEV)
    ka = workloads.make_tensor(a.shape("k"), 78, "bf16").to(DEV)
    qb = torch.zeros(b.shape("q"), dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros(b.shape("k"), dtype=torch.bfloat16, device=DEV)
    L = a.lengths
    for s in range(8):
        qb[2048 * s: 2048 * s + L[s]] = qa[a.cu_seqlens[s]: a.cu_seqlens[s + 1]]
        kb[2048 * s: 2048 * s + L[s]] = ka[a.cu_seqlens[s]: a.cu_seqlens[s + 1]]
    rope.qk_fwd_(qa, ka, torch.from_numpy(a.cu_seqlens).to(DEV), a.theta)
    rope.qk_fwd_(qb, kb, torch.from_numpy(b.cu_seqlens).to(DEV), b.theta,
                 seqused=torch.from_numpy(b.seqused).to(DEV))
    for s in range(8):
        assert torch.equal(qb[2048 * s: 2048 * s + L[s]], qa[a.cu_seqlens[s]: a.cu_seqlens[s + 1]])
        assert torch.equal(kb[2048 * s: 2048 * s + L[s]], ka[a.cu_seqlens[s]: a.cu_seqlens[s + 1]])
        assert torch.count_nonzero(qb[2048 * s + L[s]: 2048 * (s + 1)]) == 0


def test_long_context_full(rope):
    """524288 tokens, Q = 2^31 elements: the int64 path, at full size, in the launch
    configuration of a plain fwd/bwd call, checked against the oracle on every
    element of Q, K, dQ and dK (in chunks of 32768 tokens)."""
    w = workloads.get("long_ctx_512k")
    print("[parity] long_ctx_512k full (int64 path)", flush=True)
    dev = {what: workloads.make_tensor(w.shape(what), w.seed(what), "bf16", device=DEV,
                                       chunk_rows=32768)
           for what in ("q", "k", "dq", "dk")}
    before = {what: bits(t) for what, t in dev.items()}  # host copies of the inputs
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    rope.qk_fwd_(dev["q"], dev["k"], cu, w.theta)
    rope.qk_bwd_(dev["dq"], dev["dk"], cu, w.theta)
    torch.cuda.synchronize()
    chunk = 32768
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        for a in range(0, w.T, chunk):
            b = min(w.T, a + chunk)
            tokens = np.arange(a, b, dtype=np.int64)
            x = np.ascontiguousarray(before[what][a:b])
            got = bits(dev[what][a:b])
            ref = oracle.rope_rows(x, tokens, w.cu_seqlens, w.theta, direction, "bf16", None,
                                   NTHREADS)
            assert_parity("bf16", got, ref, x, np.ones(b - a, dtype=bool),
                          f"long_ctx:{what}[{a}:{b}]")
        print(f"[parity] long_ctx_512k {what}: all {w.T} tokens checked", flush=True)
    pos, seq = rope.positions(cu, w.T)
    assert torch.equal(pos, torch.arange(w.T, dtype=torch.int32, device=DEV))
    assert int(seq.min()) == 0 and int(seq.max()) == 0
    del dev, before
    torch.cuda.empty_cache()


# ------------------------------------------------- passes issued as several launches
# A long pass of the row-group kernel on a Q-heavy head shape goes out as several
# launches over consecutive token ranges (bench.group_pieces mirrors the rule); these
# cases cross the range boundaries with sequences, offsets and untouched tokens.

def _guarded_dev(t: torch.Tensor, guard: int = 4096):
    """A copy of device tensor t inside a larger buffer whose guard regions hold canaries."""
    n = t.numel()
    flat = torch.empty(n + 2 * guard, dtype=t.dtype, device=DEV)
    flat.view(_word(t.dtype)).fill_(_canary(t.dtype))
    view = flat[guard:guard + n].view(t.shape)
    view.copy_(t)
    return view, flat, guard


def _piece_marks(pieces, T, width=8):
    """Tokens on both sides of every boundary between the launches of a pass."""
    edges = np.cumsum(pieces)[:-1]
    marks = np.concatenate([np.arange(e - width, e + width) for e in edges] +
                           [np.arange(0, 16), np.arange(T - 16, T)])
    return marks[(marks >= 0) & (marks < T)]


def test_split_pass_ragged_full(rope):
    """32 + 8 heads, bf16, 200003 rows: 4 launches over 50008, 50008, 50008 and 49979
    tokens. Sequences start on, next to and across the range boundaries, and the last
    13 rows lie past cu_seqlens' end (untouched). Every element of Q, K, dQ and dK
    against the oracle; guard regions intact."""
    import bench
    T, Hq, Hkv, D = 200003, 32, 8, 128
    w = workloads.Workload("split", 92, T, Hq, Hkv, D, "bf16", 1e6,
                           np.array([0, T], dtype=np.int32))
    pieces = bench.group_pieces(T, w)
    assert pieces == [50008, 50008, 50008, 49979]
    rng = np.random.default_rng(9600)
    cuts = set(rng.integers(1, T - 13, 12).tolist()) | {50008, 100017, 150023, 150024}
    cu_h = np.array([0, *sorted(cuts), T - 13], dtype=np.int32)
    print(f"[parity] split pass, {len(cu_h) - 1} sequences, pieces {pieces}", flush=True)
    cu = torch.from_numpy(cu_h).to(DEV)
    dev, flats = {}, {}
    for i, what in enumerate(("q", "k", "dq", "dk")):
        shape = (T, Hq if what in ("q", "dq") else Hkv, D)
        t = workloads.make_tensor(shape, 9610 + i, "bf16", device=DEV, chunk_rows=32768)
        dev[what], flats[what], g = _guarded_dev(t)
        del t
    before = {what: bits(t) for what, t in dev.items()}
    rope.qk_fwd_(dev["q"], dev["k"], cu, 1e6)
    rope.qk_bwd_(dev["dq"], dev["dk"], cu, 1e6)
    torch.cuda.synchronize()
    pos, _ = oracle.positions(cu_h, T)
    chunk = 32768
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        assert guards_intact(flats[what], g), f"split:{what}: guard region written"
        for a in range(0, T, chunk):
            b = min(T, a + chunk)
            tokens = np.arange(a, b, dtype=np.int64)
            x = np.ascontiguousarray(before[what][a:b])
            ref = oracle.rope_rows(x, tokens, cu_h, 1e6, direction, "bf16", None, NTHREADS)
            assert_parity("bf16", bits(dev[what][a:b]), ref, x, pos[a:b] >= 0,
                          f"split:{what}[{a}:{b}]")
    del dev, flats, before
    torch.cuda.empty_cache()


SPLIT_CASES = [  # name, T, Hq, Hkv, dtype, expected pieces
    ("cu", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
    ("offsets", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
    ("ids", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
    ("scale", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
    ("table", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
    ("f32", 70000, 32, 8, "f32", [23336, 23336, 23328]),
    ("f16", 73000, 64, 8, "f16", [24336, 24336, 24328]),
    ("int64", 73000, 64, 8, "bf16", [24336, 24336, 24328]),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_pass_position_sources(rope, case):
    """Passes issued as several launches with every position source (cu_seqlens alone,
    per-sequence offsets, explicit ids with untouched tokens, linear scaling, cos/sin
    tables), fp32 and fp16 storage, and 64-bit offsets forced: the whole tensors bit
    for bit against the token kernel (tokens_per_wave=1, never split) and sampled
    rows (both sides of every launch boundary, random rows) against the oracle."""
    import bench
    name, T, Hq, Hkv, dtype, expect = case
    D, theta = 128, 1e6
    w = workloads.Workload("split", 93, T, Hq, Hkv, D, dtype, theta,
                           np.array([0, T], dtype=np.int32))
    pieces = bench.group_pieces(T, w)
    assert pieces == expect
    print(f"[parity] split pass {name}: T={T} {Hq}+{Hkv} {dtype} pieces {pieces}", flush=True)
    rng = np.random.default_rng(9700)
    cu_h = np.array([0, *sorted(set(rng.integers(1, T, 9).tolist()) | {pieces[0] + 3}), T],
                    dtype=np.int32)
    B = len(cu_h) - 1
    offs_h = rng.integers(0, 400000, B).astype(np.int32) if name == "offsets" else None
    ids_h = None
    if name == "ids":
        ids_h = rng.integers(0, 500000, T).astype(np.int32)
        ids_h[rng.choice(T, 2000, replace=False)] = -1
        ids_h[pieces[0] - 2:pieces[0] + 2] = [-1, 7, -1, 524287]
    scale = 4.0 if name == "scale" else 1.0
    cu = torch.from_numpy(cu_h).to(DEV)
    offs = None if offs_h is None else torch.from_numpy(offs_h).to(DEV)
    ids = None if ids_h is None else torch.from_numpy(ids_h).to(DEV)
    src = {what: workloads.make_tensor((T, Hq if what in ("q", "dq") else Hkv, D), 9710 + i,
                                       dtype, device=DEV, chunk_rows=32768)
           for i, what in enumerate(("q", "k", "dq", "dk"))}
    marks = _piece_marks(pieces, T)
    tokens = np.unique(np.concatenate([marks, rng.integers(0, T, 2048)]))
    tok_dev = torch.from_numpy(tokens).to(DEV)
    tables = None
    if name == "table":
        tables = rope.cos_sin_table(int(np.diff(cu_h).max()), D, theta, DEV)

    index_mode = rope.INDEX_64 if name == "int64" else rope.INDEX_AUTO

    def apply(q, k, direction, **kw):
        if tables is not None and not kw:
            rope.qk_apply_table_(q, k, tables[0], tables[1], direction, cu_seqlens=cu)
            return
        rope.qk_apply_ex_(q, k, theta, direction, cu_seqlens=None if ids is not None else cu,
                          seq_offsets=offs, position_ids=ids, pos_scale=scale,
                          index_mode=index_mode, **kw)

    for fwd, grad, direction in (("q", "k", 1), ("dq", "dk", -1)):
        a_q, a_k = src[fwd].clone(), src[grad].clone()
        b_q, b_k = src[fwd].clone(), src[grad].clone()
        apply(a_q, a_k, direction)
        apply(b_q, b_k, direction, tokens_per_wave=1)
        torch.cuda.synchronize()
        assert torch.equal(a_q.view(_word(a_q.dtype)), b_q.view(_word(b_q.dtype))), (name, fwd)
        assert torch.equal(a_k.view(_word(a_k.dtype)), b_k.view(_word(b_k.dtype))), (name, grad)
        for what, got_t in ((fwd, a_q), (grad, a_k)):
            x = bits(src[what].index_select(0, tok_dev))
            got = bits(got_t.index_select(0, tok_dev))
            if ids_h is not None:
                ref = oracle.rope_rows(x, tokens, None, theta, direction, dtype, None, NTHREADS,
                                       position_ids=ids_h)
                touched = ids_h[tokens] >= 0
            else:
                ref = oracle.rope_rows(x, tokens, cu_h, theta, direction, dtype, None, NTHREADS,
                                       seq_offsets=offs_h, pos_scale=scale)
                touched = np.ones(len(tokens), dtype=bool)
            assert_parity(dtype, got, ref, x, touched, f"split-{name}:{what}")
        del a_q, a_k, b_q, b_k
    del src
    torch.cuda.empty_cache()


def test_split_pass_fused_qkv_views(rope):
    """A pass issued as several launches on Q and K as strided views into fused QKV
    outputs (73000 tokens, 64 + 8 heads: 3 launches): bit for bit the token kernel on
    the same views, forward and backward, V untouched."""
    T, Hq, Hkv, D = 73000, 64, 8, 128
    print("[parity] split pass on fused qkv views", flush=True)
    qkv0 = workloads.make_tensor((T, (Hq + 2 * Hkv) * D), 9800, "bf16", device=DEV, chunk_rows=8192)
    cu = torch.tensor([0, 30000, 48670, T], dtype=torch.int32, device=DEV)
    a, b = qkv0.clone(), qkv0.clone()
    for direction in (1, -1):
        qa, ka, _ = _qkv_views(a, Hq, Hkv, D)
        qb, kb, _ = _qkv_views(b, Hq, Hkv, D)
        rope.qk_apply_ex_(qa, ka, 1e6, direction, cu_seqlens=cu)
        rope.qk_apply_ex_(qb, kb, 1e6, direction, cu_seqlens=cu, tokens_per_wave=1)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), direction
        if direction == 1:  # the forward rotated the last token range too
            assert not torch.equal(a[-100:].view(torch.int16), qkv0[-100:].view(torch.int16))
    _, _, v = _qkv_views(a, Hq, Hkv, D)
    _, _, v0 = _qkv_views(qkv0, Hq, Hkv, D)
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16))
    del qkv0, a, b
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- exports

@pytest.mark.parametrize("name", workloads.names())
def test_positions_export(rope, name):
    w = workloads.get(name)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = None if w.seqused is None else torch.from_numpy(w.seqused).to(DEV)
    pos, seq = rope.positions(cu, w.T, su)
    rpos, rseq = oracle.positions(w.cu_seqlens, w.T, w.seqused)
    assert np.array_equal(pos.cpu().numpy(), rpos) and np.array_equal(seq.cpu().numpy(), rseq)


def test_positions_edges(rope):
    cases = [([2, 2, 5, 9], [0, 2, 9], 11), ([0, 0, 0], None, 3), ([0, 7], None, 12),
             ([3, 3, 3, 10, 10, 11], [1, 0, 4, 0, 1], 16), ([0] + list(range(1, 300)), None, 300)]
    for cu_l, su_l, T in cases:
        cu = torch.tensor(cu_l, dtype=torch.int32, device=DEV)
        su = None if su_l is None else torch.tensor(su_l, dtype=torch.int32, device=DEV)
        pos, seq = rope.positions(cu, T, su)
        rpos, rseq = oracle.positions(cu_l, T, su_l)
        assert np.array_equal(pos.cpu().numpy(), rpos), (cu_l, su_l)
        assert np.array_equal(seq.cpu().numpy(), rseq), (cu_l, su_l)


@pytest.mark.parametrize("theta,D,maxpos", [(1e4, 16, 64), (1e6, 128, 524288), (1e4, 128, 40000),
                                            (5e5, 64, 70000), (1e6, 80, 20000)])
def test_cos_sin_export_bit_exact(rope, theta, D, maxpos):
    """Both exports against the oracle's correctly rounded values: the [max_pos, D/2]
    table of positions 0 .. max_pos-1, and the same positions as a shuffled list."""
    pos = np.arange(maxpos, dtype=np.int32)
    rc, rs = oracle.cos_sin(pos, D, theta)
    perm = np.random.default_rng(maxpos).permutation(maxpos).astype(np.int32)
    tc, ts = rope.cos_sin_table(maxpos, D, theta, DEV)
    lc, ls = rope.cos_sin(torch.from_numpy(perm).to(DEV), D, theta)
    for form, c, s, rows in (("table", tc, ts, pos), ("list", lc, ls, perm)):
        cb, sb = c.cpu().numpy().view(np.uint32), s.cpu().numpy().view(np.uint32)
        mism = int((cb != rc[rows].view(np.uint32)).sum() + (sb != rs[rows].view(np.uint32)).sum())
        assert mism == 0, f"{form}: {mism} of {2 * rc.size} cos/sin values differ from the oracle"


def test_positions_without_sequences(rope):
    """num_seqs == 0 with no cu_seqlens (NULL) and no ids: every token is untouched
    (-1) and nothing is read from the missing array."""
    T = 1000
    pos = torch.full((T,), 7, dtype=torch.int32, device=DEV)
    seq = torch.full((T,), 7, dtype=torch.int32, device=DEV)
    st = rope._lib.rope_positions_ex(None, 0, None, None, None, T, pos.data_ptr(),
                                     seq.data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0
    st = rope._lib.rope_positions(None, 0, None, T, pos.data_ptr(), None,
                                  torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert bool(torch.all(pos == -1)) and bool(torch.all(seq == -1))


# ---------------------------------------------------------------- launch variants

@pytest.mark.parametrize("name", ["tiny_packed", "qwen3_4b_packed"])
def test_variants_bit_identical(rope, name):
    """int64 indexing forced, and several launch geometries: same bits as default."""
    w = workloads.get(name)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    q0 = workloads.make_tensor(w.shape("q"), w.seed("q"), w.dtype).to(DEV)
    k0 = workloads.make_tensor(w.shape("k"), w.seed("k"), w.dtype).to(DEV)
    q_ref, k_ref = q0.clone(), k0.clone()
    rope.qk_fwd_(q_ref, k_ref, cu, w.theta)
    for kw in (dict(index_mode=rope.INDEX_64), dict(index_mode=rope.INDEX_32),
               dict(tokens_per_wave=1), dict(tokens_per_wave=3), dict(tokens_per_wave=8),
               dict(tokens_per_wave=min(w.T, 1024)), dict(tokens_per_wave=1024),
               dict(index_mode=rope.INDEX_64, tokens_per_wave=5)):
        print(f"[parity] {name} variant {kw}", flush=True)
        q, k = q0.clone(), k0.clone()
        rope.qk_apply_(q, k, cu, w.theta, 1, **kw)
        assert torch.equal(q.view(torch.int16 if w.dtype != "f32" else torch.int32),
                           q_ref.view(torch.int16 if w.dtype != "f32" else torch.int32)), kw
        assert torch.equal(k, k_ref), kw


@pytest.mark.parametrize("name", ["qwen3_8b_packed", "qwen3_8b_padded", "qwen3_32b_packed"])
def test_int64_forced_bit_identical(rope, name):
    """The 64-bit offset specialization forced on the workloads that select 32-bit
    offsets by default (the packed and padded comparison batches and the Qwen3-32B
    shape) gives the same bits, forward and backward."""
    w = workloads.get(name)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = None if w.seqused is None else torch.from_numpy(w.seqused).to(DEV)
    word = torch.int16 if w.dtype != "f32" else torch.int32
    for direction, (a, b) in ((1, ("q", "k")), (-1, ("dq", "dk"))):
        print(f"[parity] {name} forced int64, direction {direction}", flush=True)
        x0 = workloads.make_tensor(w.shape(a), w.seed(a), w.dtype).to(DEV)
        y0 = workloads.make_tensor(w.shape(b), w.seed(b), w.dtype).to(DEV)
        xr, yr = x0.clone(), y0.clone()
        rope.qk_apply_(xr, yr, cu, w.theta, direction, seqused=su)
        x, y = x0.clone(), y0.clone()
        rope.qk_apply_(x, y, cu, w.theta, direction, seqused=su, index_mode=rope.INDEX_64)
        torch.cuda.synchronize()
        assert torch.equal(x.view(word), xr.view(word)), (name, direction, a)
        assert torch.equal(y.view(word), yr.view(word)), (name, direction, b)
        assert not torch.equal(xr.view(word), x0.view(word))  # the launch did rotate


# ---------------------------------------------------------------- edge cases

EDGE = [
    # (label, lengths (cu from 0 unless cu given), T, Hq, Hkv, D, dtype, theta, seqused, cu)
    ("ragged_bf16_D128", [37, 0, 300, 1, 5], 343, 3, 1, 128, "bf16", 1e6, None, None),
    ("bf16_D2_vec1", [9, 20], 29, 4, 2, 2, "bf16", 1e4, None, None),
    ("bf16_D6_vec1", [9, 20], 29, 4, 2, 6, "bf16", 1e4, None, None),
    ("bf16_D12_vec2", [30, 3], 33, 2, 2, 12, "bf16", 1e4, None, None),
    ("bf16_D40_vec4", [30, 3], 33, 2, 2, 40, "bf16", 1e4, None, None),
    ("bf16_D80_nc5", [50, 70], 120, 3, 2, 80, "bf16", 1e6, None, None),
    ("bf16_D96_nc6", [50, 70, 3], 123, 32, 8, 96, "bf16", 1e6, None, None),
    ("f16_D112_nc7", [50, 1, 70], 121, 9, 7, 112, "f16", 1e6, None, None),
    ("bf16_D160_nc10", [64, 57], 121, 13, 5, 160, "bf16", 1e6, None, None),
    ("bf16_D192_nc12", [64, 57], 121, 6, 1, 192, "bf16", 1e6, None, None),
    ("f32_D96_nc12", [30, 40], 70, 5, 3, 96, "f32", 1e4, None, None),
    ("bf16_D48_nc3", [30, 40], 70, 22, 21, 48, "bf16", 1e4, None, None),
    ("bf16_D320_nc20", [30, 40], 70, 7, 2, 320, "bf16", 1e6, None, None),
    ("bf16_D100_vec2", [30, 40], 70, 3, 2, 100, "bf16", 1e4, None, None),
    ("bf16_D256", [50, 70], 120, 3, 2, 256, "bf16", 1e6, None, None),
    ("bf16_D512_max", [50, 70], 120, 2, 1, 512, "bf16", 1e6, None, None),
    ("f32_D64", [10, 100, 17], 127, 4, 4, 64, "f32", 1e4, None, None),
    ("f32_D2", [10, 100, 17], 127, 1, 1, 2, "f32", 1e4, None, None),
    ("f16_D128", [10, 100, 17], 127, 8, 2, 128, "f16", 5e5, None, None),
    ("k_only", [40, 24], 64, 0, 4, 64, "bf16", 1e4, None, None),
    ("q_only", [40, 24], 64, 4, 0, 64, "bf16", 1e4, None, None),
    ("cu_offset_tail_seqused", None, 40, 3, 1, 32, "bf16", 1e4, [0, 5, 100, 2], [3, 3, 12, 30, 35]),
    ("many_tiny_seqs", [1] * 200 + [2] * 50, 320, 2, 2, 64, "bf16", 1e4, None, None),
    ("theta_one", [33, 31], 64, 2, 2, 64, "bf16", 1.0, None, None),
    ("heads_many", [20, 13], 33, 96, 16, 64, "bf16", 1e4, None, None),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(rope, case):
    label, lengths, T, Hq, Hkv, D, dtype, theta, su, cu = case
    if cu is None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = np.asarray(cu, dtype=np.int32)
    su = None if su is None else np.asarray(su, dtype=np.int32)
    g = 9000 + len(label)
    host = {"q": workloads.make_tensor((T, Hq, D), g, dtype),
            "k": workloads.make_tensor((T, Hkv, D), g + 1, dtype),
            "dq": workloads.make_tensor((T, Hq, D), g + 2, dtype),
            "dk": workloads.make_tensor((T, Hkv, D), g + 3, dtype)}
    run_and_check(rope, label, host, cu, su, theta, dtype)


STAGED_CASES = [  # (D, dtype, Hq, Hkv): row halves that are not whole 128-byte lines
    (80, "bf16", 32, 32), (96, "bf16", 32, 8), (112, "f16", 28, 4), (160, "bf16", 16, 16),
    (48, "bf16", 40, 8), (64, "bf16", 32, 8), (32, "bf16", 16, 4), (16, "f32", 8, 8),
    (64, "f16", 12, 2), (112, "bf16", 20, 4), (48, "f16", 27, 3), (144, "bf16", 14, 2),
]


@pytest.mark.parametrize("case", STAGED_CASES, ids=[f"{c[1]}_D{c[0]}" for c in STAGED_CASES])
def test_staged_chunk_count(rope, case):
    """The row-group kernel's staged instance (a group of group_rows(nc) rows, e.g. 8
    for D = 112, 20 for D = 48, 7 for D = 144, moved through LDS in whole lines): bit
    for bit the token kernel with cu_seqlens, per-sequence offsets, explicit ids,
    64-bit offsets forced and cos/sin tables, forward and backward, on 3000 tokens in
    ragged sequences; sampled rows against the oracle."""
    _check_group_instance(rope, case, "staged")


ROW_STEP_CASES = [  # (D, dtype, Hq, Hkv): two row steps per workgroup
    (512, "bf16", 7, 3), (512, "f16", 8, 8), (512, "f32", 5, 3), (512, "bf16", 1, 1),
    # staged, 11 to 15 chunks per half row
    (192, "bf16", 13, 3), (176, "f16", 16, 16), (96, "f32", 11, 3), (240, "bf16", 9, 1),
    (208, "bf16", 8, 8),
]


@pytest.mark.parametrize("case", ROW_STEP_CASES, ids=[f"{c[1]}_D{c[0]}_{c[2]}x{c[3]}"
                                                      for c in ROW_STEP_CASES])
def test_row_steps(rope, case):
    """The row-group kernel with two row steps per workgroup (D = 512: 4 rows per
    workgroup in 16-bit storage, 2 in fp32; the staged instance at 11 to 15 chunks
    per half row: 10 rows for D = 192 and fp32 D = 96, 8 for D = 176, 208 and 240; head counts that end inside a step and inside a group): the same checks
    as the staged instance."""
    _check_group_instance(rope, case, "row steps")


def _check_group_instance(rope, case, label):
    D, dtype, Hq, Hkv = case
    T = 3000
    print(f"[parity] {label} D={D} {dtype} {Hq}+{Hkv}", flush=True)
    rng = np.random.default_rng(9900 + D)
    cu_h = np.array([0, 1, 700, 701, 2100, 2999, T], dtype=np.int32)
    cu = torch.from_numpy(cu_h).to(DEV)
    offs_h = rng.integers(0, 100000, len(cu_h) - 1).astype(np.int32)
    offs = torch.from_numpy(offs_h).to(DEV)
    ids_h = rng.integers(0, 70000, T).astype(np.int32)
    ids_h[rng.choice(T, 100, replace=False)] = -1
    ids = torch.from_numpy(ids_h).to(DEV)
    tables = rope.cos_sin_table(int(np.diff(cu_h).max()), D, 1e6, DEV)
    src = {what: workloads.make_tensor((T, Hq if what in ("q", "dq") else Hkv, D), 9910 + i,
                                       dtype, device=DEV)
           for i, what in enumerate(("q", "k", "dq", "dk"))}
    modes = {
        "cu": dict(cu_seqlens=cu),
        "offsets": dict(cu_seqlens=cu, seq_offsets=offs),
        "ids": dict(position_ids=ids),
        "int64": dict(cu_seqlens=cu, index_mode=rope.INDEX_64),
    }
    word = _word(src["q"].dtype)
    tokens = np.unique(np.concatenate([np.arange(0, 8), np.arange(T - 8, T),
                                       rng.integers(0, T, 200)]))
    tok_dev = torch.from_numpy(tokens).to(DEV)
    for fwd, grad, direction in (("q", "k", 1), ("dq", "dk", -1)):
        for mode, kw in modes.items():
            a_q, a_k = src[fwd].clone(), src[grad].clone()
            b_q, b_k = src[fwd].clone(), src[grad].clone()
            rope.qk_apply_ex_(a_q, a_k, 1e6, direction, **kw)
            rope.qk_apply_ex_(b_q, b_k, 1e6, direction, tokens_per_wave=1, **kw)
            torch.cuda.synchronize()
            assert torch.equal(a_q.view(word), b_q.view(word)), (mode, fwd)
            assert torch.equal(a_k.view(word), b_k.view(word)), (mode, grad)
            for what, got_t in ((fwd, a_q), (grad, a_k)):
                x = bits(src[what].index_select(0, tok_dev))
                got = bits(got_t.index_select(0, tok_dev))
                if mode == "ids":
                    ref = oracle.rope_rows(x, tokens, None, 1e6, direction, dtype, None,
                                           NTHREADS, position_ids=ids_h)
                    touched = ids_h[tokens] >= 0
                else:
                    ref = oracle.rope_rows(x, tokens, cu_h, 1e6, direction, dtype, None,
                                           NTHREADS, seq_offsets=offs_h if mode == "offsets"
                                           else None)
                    touched = np.ones(len(tokens), dtype=bool)
                assert_parity(dtype, got, ref, x, touched, f"{label}-{mode}:{what}")
        t_q, t_k = src[fwd].clone(), src[grad].clone()
        c_q, c_k = src[fwd].clone(), src[grad].clone()
        rope.qk_apply_table_(t_q, t_k, tables[0], tables[1], direction, cu_seqlens=cu)
        rope.qk_apply_ex_(c_q, c_k, 1e6, direction, cu_seqlens=cu)
        torch.cuda.synchronize()
        assert torch.equal(t_q.view(word), c_q.view(word)) and torch.equal(t_k.view(word),
                                                                            c_k.view(word))


def test_staged_on_fused_qkv_views(rope):
    """The staged instance on Q and K as strided views into fused QKV outputs (D = 96,
    bf16, 32 + 8 heads, 4000 tokens): bit for bit the token kernel on the same views,
    forward and backward, V untouched."""
    T, Hq, Hkv, D = 4000, 32, 8, 96
    print("[parity] staged on fused qkv views", flush=True)
    qkv0 = workloads.make_tensor((T, (Hq + 2 * Hkv) * D), 9960, "bf16", device=DEV)
    cu = torch.tensor([0, 1500, 1501, T], dtype=torch.int32, device=DEV)
    a, b = qkv0.clone(), qkv0.clone()
    for direction in (1, -1):
        qa, ka, _ = _qkv_views(a, Hq, Hkv, D)
        qb, kb, _ = _qkv_views(b, Hq, Hkv, D)
        rope.qk_apply_ex_(qa, ka, 1e6, direction, cu_seqlens=cu)
        rope.qk_apply_ex_(qb, kb, 1e6, direction, cu_seqlens=cu, tokens_per_wave=1)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), direction
        if direction == 1:
            assert not torch.equal(a.view(torch.int16), qkv0.view(torch.int16))
    _, _, v = _qkv_views(a, Hq, Hkv, D)
    _, _, v0 = _qkv_views(qkv0, Hq, Hkv, D)
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16))


@pytest.mark.parametrize("D", [96, 112])
def test_staged_chunk_count_split_and_compact(rope, D):
    """The staged instance (bf16, 32 + 8 heads; D = 96: 10 rows per group, D = 112:
    8 rows, whole lines; 4 + 1 groups per token either way) in a pass issued as 2
    launches (131072 tokens) and in a compact padded launch: bit for bit the token
    kernel, sampled rows against the oracle."""
    import bench
    T, Hq, Hkv = 131072, 32, 8
    w = workloads.Workload("g", 94, T, Hq, Hkv, D, "bf16", 1e6, np.array([0, T], dtype=np.int32))
    assert bench.group_pieces(T, w) == [65536, 65536]
    print(f"[parity] staged D={D}, split pass and compact launch", flush=True)
    cu_h = np.array([0, 65530, 65541, T], dtype=np.int32)
    cu = torch.from_numpy(cu_h).to(DEV)
    q0 = workloads.make_tensor((T, Hq, D), 9950, "bf16", device=DEV, chunk_rows=32768)
    k0 = workloads.make_tensor((T, Hkv, D), 9951, "bf16", device=DEV, chunk_rows=32768)
    a_q, a_k, b_q, b_k = q0.clone(), k0.clone(), q0.clone(), k0.clone()
    rope.qk_fwd_(a_q, a_k, cu, 1e6)
    rope.qk_apply_ex_(b_q, b_k, 1e6, 1, cu_seqlens=cu, tokens_per_wave=1)
    torch.cuda.synchronize()
    assert torch.equal(a_q.view(torch.int16), b_q.view(torch.int16))
    assert torch.equal(a_k.view(torch.int16), b_k.view(torch.int16))
    tokens = np.unique(np.concatenate([np.arange(65520, 65560), np.arange(T - 8, T),
                                       np.arange(0, T, 997)]))
    tok_dev = torch.from_numpy(tokens).to(DEV)
    x = bits(q0.index_select(0, tok_dev))
    ref = oracle.rope_rows(x, tokens, cu_h, 1e6, 1, "bf16", None, NTHREADS)
    assert_parity("bf16", bits(a_q.index_select(0, tok_dev)), ref, x,
                  np.ones(len(tokens), bool), "staged-split:q")
    # compact: 8 sequences padded to 16384 rows, 40-100% used
    S, B = 16384, 8
    cu_p = torch.from_numpy((np.arange(B + 1) * S).astype(np.int32)).to(DEV)
    su_h = np.array([16384, 9000, 6554, 16000, 12345, 7000, 8191, 16383], dtype=np.int32)
    su = torch.from_numpy(su_h).to(DEV)
    cv = rope.valid_prefix(cu_p, su)
    c_q, c_k, d_q, d_k = q0.clone(), k0.clone(), q0.clone(), k0.clone()
    rope.qk_apply_padded_(c_q, c_k, 1e6, -1, cu_p, su, cv, int(su_h.sum()))
    rope.qk_apply_ex_(d_q, d_k, 1e6, -1, cu_seqlens=cu_p, seqused=su)
    torch.cuda.synchronize()
    assert torch.equal(c_q.view(torch.int16), d_q.view(torch.int16))
    assert torch.equal(c_k.view(torch.int16), d_k.view(torch.int16))
    del q0, k0, a_q, a_k, b_q, b_k, c_q, c_k, d_q, d_k
    torch.cuda.empty_cache()


def test_misaligned_views(rope):
    """Views that start 1 element off a 16-byte boundary take the narrow-access path."""
    T, Hq, Hkv, D = 50, 3, 2, 128
    cu = np.array([0, 20, 50], dtype=np.int32)
    print("[parity] misaligned views", flush=True)
    buf_q = torch.empty(T * Hq * D + 1, dtype=torch.bfloat16, device=DEV)
    buf_k = torch.empty(T * Hkv * D + 1, dtype=torch.bfloat16, device=DEV)
    q = buf_q[1:].view(T, Hq, D)
    k = buf_k[1:].view(T, Hkv, D)
    hq = workloads.make_tensor((T, Hq, D), 31, "bf16")
    hk = workloads.make_tensor((T, Hkv, D), 32, "bf16")
    q.copy_(hq)
    k.copy_(hk)
    assert q.data_ptr() % 16 != 0
    rope.qk_fwd_(q, k, torch.from_numpy(cu).to(DEV), 1e6)
    torch.cuda.synchronize()
    touched = np.ones(T, dtype=bool)
    for name, dv, hv, H in (("q", q, hq, Hq), ("k", k, hk, Hkv)):
        ref = oracle.rope(bits(hv), cu, 1e6, 1, "bf16")
        assert_parity("bf16", bits(dv), ref, bits(hv), touched, f"misaligned:{name}")


def test_bwd_after_fwd_is_identity_fp32(rope):
    w = workloads.get("tiny_packed")
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    x = workloads.make_tensor((w.T, w.Hq, w.D), 5, "f32").to(DEV)
    y = workloads.make_tensor((w.T, w.Hkv, w.D), 6, "f32").to(DEV)
    q, k = x.clone(), y.clone()
    rope.qk_fwd_(q, k, cu, w.theta)
    assert not torch.equal(q, x)
    rope.qk_bwd_(q, k, cu, w.theta)
    assert torch.max(torch.abs(q - x)) <= 8 * 2.0 ** -24 * torch.max(torch.abs(x))
    assert torch.max(torch.abs(k - y)) <= 8 * 2.0 ** -24 * torch.max(torch.abs(y))


def test_binding_rejects_bad_tensors(rope):
    cu = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    q = torch.zeros(4, 2, 8, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(4, 1, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        rope.qk_fwd_(q, k.float(), cu, 1e4)
    with pytest.raises(ValueError):
        rope.qk_fwd_(q.transpose(0, 1), k, cu, 1e4)
    with pytest.raises(TypeError):
        rope.qk_fwd_(q, k, cu.long(), 1e4)
    with pytest.raises(rope.RopeError):
        rope.qk_fwd_(q, k, cu, 0.5)
    with pytest.raises(rope.RopeError):
        rope.qk_fwd_(torch.zeros(4, 2, 7, dtype=torch.bfloat16, device=DEV),
                     torch.zeros(4, 1, 7, dtype=torch.bfloat16, device=DEV), cu, 1e4)


# ---------------------------------------------------------------- NEXT rows: explicit
# position ids, per-sequence offsets, linear position interpolation

def test_position_ids_parity(rope):
    """Explicit per-token positions (negative = untouched), forward and backward, on the
    Qwen3-4B-shaped batch, against the oracle."""
    w = workloads.get("qwen3_4b_packed")
    print("[parity] position_ids on qwen3_4b_packed", flush=True)
    rng = np.random.default_rng(77)
    ids = rng.integers(0, 40960, w.T).astype(np.int32)
    ids[rng.choice(w.T, 500, replace=False)] = -1
    ids[:5] = [0, 1, 2, 40959, 2 ** 31 - 1]
    host = make_host(w, canary_untouched=False)
    dev = {k: v.to(DEV) for k, v in host.items()}
    pid = torch.from_numpy(ids).to(DEV)
    rope.qk_fwd_pos_(dev["q"], dev["k"], pid, w.theta)
    rope.qk_bwd_pos_(dev["dq"], dev["dk"], pid, w.theta)
    torch.cuda.synchronize()
    touched = ids >= 0
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        x = bits(host[what])
        ref = oracle.rope(x, None, w.theta, direction, "bf16", nthreads=NTHREADS, position_ids=ids)
        assert_parity("bf16", bits(dev[what]), ref, x, touched, f"ids:{what}")
    pos, seq = rope.positions(None, w.T, position_ids=pid)
    rpos, rseq = oracle.positions(None, w.T, position_ids=ids)
    assert np.array_equal(pos.cpu().numpy(), rpos) and np.array_equal(seq.cpu().numpy(), rseq)


def test_seq_offsets_context_parallel_shards(rope):
    """The 524288-token sequence cut into 4 shards of 131072 tokens (one rank's share of
    4-way context parallelism), each rotated alone with the global position of its first
    token as offset: bit-identical to the unsharded result, forward and backward, and
    sampled rows of the last shard against the oracle."""
    w = workloads.get("long_ctx_512k")
    print("[parity] long_ctx_512k as 4 context-parallel shards", flush=True)
    q0 = workloads.make_tensor(w.shape("q"), w.seed("q"), "bf16", device=DEV, chunk_rows=32768)
    k0 = workloads.make_tensor(w.shape("k"), w.seed("k"), "bf16", device=DEV, chunk_rows=32768)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    for direction in (1, -1):
        qf, kf = q0.clone(), k0.clone()
        rope.qk_apply_(qf, kf, cu, w.theta, direction)
        qs, ks = q0.clone(), k0.clone()
        n = w.T // 4
        for r in range(4):
            a = r * n
            cu_r = torch.tensor([0, n], dtype=torch.int32, device=DEV)
            off = torch.tensor([a], dtype=torch.int32, device=DEV)
            rope.qk_apply_ex_(qs[a:a + n], ks[a:a + n], w.theta, direction, cu_seqlens=cu_r,
                              seq_offsets=off)
        torch.cuda.synchronize()
        assert torch.equal(qs.view(torch.int16), qf.view(torch.int16)), direction
        assert torch.equal(ks.view(torch.int16), kf.view(torch.int16)), direction
        del qs, ks
    # Sampled rows of the last shard, as that rank computes them (qf holds the last
    # direction of the loop: the backward), against the oracle.
    tokens = np.arange(3 * n, 3 * n + 64)
    tok_dev = torch.from_numpy(tokens).to(DEV)
    x = bits(q0.index_select(0, tok_dev))
    ref = oracle.rope_rows(x, tokens - 3 * n, [0, n], w.theta, -1, "bf16", None, NTHREADS,
                           seq_offsets=[3 * n])
    assert_parity("bf16", bits(qf.index_select(0, tok_dev)), ref, x, np.ones(64, bool), "cp:q")
    del q0, k0, qf, kf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pos_scale", [4.0, 2.5])
def test_pos_scale_parity(rope, pos_scale):
    """Linear position interpolation on the Qwen3-8B packed batch (bf16) against the
    oracle, and the cos/sin export at that factor bit for bit."""
    w = workloads.get("qwen3_8b_packed")
    print(f"[parity] pos_scale={pos_scale} on qwen3_8b_packed", flush=True)
    host = make_host(w, canary_untouched=False)
    dev = {k: v.to(DEV) for k, v in host.items()}
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    rope.qk_apply_ex_(dev["q"], dev["k"], w.theta, 1, cu_seqlens=cu, pos_scale=pos_scale)
    rope.qk_apply_ex_(dev["dq"], dev["dk"], w.theta, -1, cu_seqlens=cu, pos_scale=pos_scale)
    torch.cuda.synchronize()
    touched = np.ones(w.T, dtype=bool)
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        x = bits(host[what])
        ref = oracle.rope(x, w.cu_seqlens, w.theta, direction, "bf16", nthreads=NTHREADS,
                          pos_scale=pos_scale)
        assert_parity("bf16", bits(dev[what]), ref, x, touched, f"scale:{what}")
    pos = np.arange(0, 163840, 7, dtype=np.int32)
    c, s = rope.cos_sin(torch.from_numpy(pos).to(DEV), 128, 1e6, pos_scale)
    rc, rs = oracle.cos_sin(pos, 128, 1e6, pos_scale)
    assert np.array_equal(c.cpu().numpy().view(np.uint32), rc.view(np.uint32))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_positions_export_offsets(rope):
    cases = [([0, 5, 22, 25, 64], None, [100, 0, -3, 7], 64),
             ([2, 2, 5, 9], [0, 2, 9], [0, 5, -1], 11),
             ([0, 10], None, [2 ** 31 - 5], 10)]
    for cu_l, su_l, off_l, T in cases:
        cu = torch.tensor(cu_l, dtype=torch.int32, device=DEV)
        su = None if su_l is None else torch.tensor(su_l, dtype=torch.int32, device=DEV)
        off = torch.tensor(off_l, dtype=torch.int32, device=DEV)
        pos, seq = rope.positions(cu, T, su, seq_offsets=off)
        rpos, rseq = oracle.positions(cu_l, T, su_l, seq_offsets=off_l)
        assert np.array_equal(pos.cpu().numpy(), rpos), (cu_l, off_l)
        assert np.array_equal(seq.cpu().numpy(), rseq), (cu_l, off_l)


# ---------------------------------------------------------------- strided (fused QKV) views

def _qkv_views(qkv: torch.Tensor, Hq: int, Hkv: int, D: int, lead: int = 0):
    """q, k, v views [T, H, D] into a fused projection output [T, width] whose
    columns are [lead gap | Q | K | V | trailing gap]."""
    T = qkv.shape[0]
    q = qkv[:, lead:lead + Hq * D].view(T, Hq, D)
    k = qkv[:, lead + Hq * D:lead + (Hq + Hkv) * D].view(T, Hkv, D)
    v = qkv[:, lead + (Hq + Hkv) * D:lead + (Hq + 2 * Hkv) * D].view(T, Hkv, D)
    return q, k, v


@pytest.mark.parametrize("direction", [1, -1])
def test_fused_qkv_views_qwen3_8b(rope, direction):
    """Q and K rotated in place as views into the fused QKV output of the Qwen3-8B
    packed batch (token stride (32 + 2*8) * 128): bit-identical to rotating
    contiguous copies, V untouched, and against the oracle."""
    w = workloads.get("qwen3_8b_packed")
    Hq, Hkv, D = w.Hq, w.Hkv, w.D
    print(f"[parity] fused qkv views qwen3_8b_packed direction={direction}", flush=True)
    qkv0 = workloads.make_tensor((w.T, (Hq + 2 * Hkv) * D), 9100, "bf16", device=DEV)
    qkv = qkv0.clone()
    q, k, v = _qkv_views(qkv, Hq, Hkv, D)
    assert not q.is_contiguous() and q.stride(0) == (Hq + 2 * Hkv) * D
    qc, kc = q.contiguous(), k.contiguous()
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    rope.qk_apply_ex_(q, k, w.theta, direction, cu_seqlens=cu)
    rope.qk_apply_(qc, kc, cu, w.theta, direction)
    torch.cuda.synchronize()
    assert torch.equal(q.contiguous().view(torch.int16), qc.view(torch.int16))
    assert torch.equal(k.contiguous().view(torch.int16), kc.view(torch.int16))
    _, _, v0 = _qkv_views(qkv0, Hq, Hkv, D)
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16)), "V changed"
    q0, k0, _ = _qkv_views(qkv0, Hq, Hkv, D)
    touched = np.ones(w.T, dtype=bool)
    for what, x0, got in (("q", q0, q), ("k", k0, k)):
        x = bits(x0)
        ref = oracle.rope(x, w.cu_seqlens, w.theta, direction, "bf16", nthreads=NTHREADS)
        assert_parity("bf16", bits(got), ref, x, touched, f"qkv:{what}")


@pytest.mark.parametrize("dtype,D,Hq,Hkv,lead,tail", [
    (torch.float32, 64, 3, 1, 0, 2),     # stride 8 bytes past a 16-byte multiple
    (torch.float32, 96, 2, 2, 1, 0),     # base 4 bytes off: 4-byte accesses
    (torch.float16, 128, 5, 1, 0, 3),    # odd stride in 2-byte words
    (torch.bfloat16, 256, 4, 2, 8, 8),   # gaps on both sides, 16-byte aligned
    (torch.bfloat16, 2, 3, 1, 1, 1),     # smallest head dimension
])
def test_strided_views_ragged(rope, dtype, D, Hq, Hkv, lead, tail):
    """Views with leading/trailing gaps and strides that force narrower accesses, on a
    ragged batch with an empty sequence and a token tail: parity with the oracle,
    gaps and V bit-for-bit untouched."""
    name = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    lengths = [37, 0, 129, 1, 64]
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu_h[-1]) + 5  # tokens past the last sequence are left untouched
    width = lead + (Hq + 2 * Hkv) * D + tail
    print(f"[parity] strided views {name} D={D} Hq={Hq} Hkv={Hkv} lead={lead} tail={tail}",
          flush=True)
    qkv0 = workloads.make_tensor((T, width), 9200 + D, name, device=DEV)
    qkv = qkv0.clone()
    q, k, _ = _qkv_views(qkv, Hq, Hkv, D, lead)
    cu = torch.from_numpy(cu_h).to(DEV)
    rope.qk_apply_ex_(q, k, 1e4, 1, cu_seqlens=cu)
    torch.cuda.synchronize()
    q0, k0, _ = _qkv_views(qkv0, Hq, Hkv, D, lead)
    pos, _ = oracle.positions(cu_h, T)
    touched = pos >= 0
    for what, x0, got in (("q", q0, q), ("k", k0, k)):
        x = bits(x0)
        ref = oracle.rope(x, cu_h, 1e4, 1, name, nthreads=NTHREADS)
        assert_parity(name, bits(got), ref, x, touched, f"strided:{what}")
    # everything outside the Q and K views is unchanged
    mask = torch.ones(width, dtype=torch.bool, device=DEV)
    mask[lead:lead + (Hq + Hkv) * D] = False
    word = _word(dtype)
    assert torch.equal(qkv.view(word)[:, mask], qkv0.view(word)[:, mask])


def test_stride_forces_64bit_offsets(rope):
    """A token stride that takes offsets past 2^31 elements while T*H*D stays small:
    the library must switch to 64-bit offsets by itself. 8192 tokens, one head each,
    2^18 elements apart (a 4 GiB bf16 buffer); the result matches the oracle."""
    T, D, stride = 8192, 128, 1 << 18
    print("[parity] 64-bit offsets from a large token stride", flush=True)
    buf = torch.zeros((T, stride), dtype=torch.bfloat16, device=DEV)
    vals = workloads.make_tensor((T, 2, D), 9300, "bf16", device=DEV)
    buf[:, :D] = vals[:, 0]
    buf[:, stride - D:] = vals[:, 1]
    q = buf[:, :D].view(T, 1, D)
    k = buf[:, stride - D:].view(T, 1, D)
    assert q.stride(0) == stride and T * stride >= 1 << 31
    lengths = [1000, 4000, 3192]
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rope.qk_apply_ex_(q, k, 1e6, 1, cu_seqlens=torch.from_numpy(cu_h).to(DEV))
    with pytest.raises(rope.RopeError):
        rope.qk_apply_ex_(q, k, 1e6, 1, cu_seqlens=torch.from_numpy(cu_h).to(DEV),
                          index_mode=rope.INDEX_32)
    torch.cuda.synchronize()
    touched = np.ones(T, dtype=bool)
    for what, x0, got in (("q", vals[:, :1], q), ("k", vals[:, 1:], k)):
        x = bits(x0)
        ref = oracle.rope(x, cu_h, 1e6, 1, "bf16", nthreads=NTHREADS)
        assert_parity("bf16", bits(got), ref, x, touched, f"stride64:{what}")
    assert torch.count_nonzero(buf[:, D:stride - D]).item() == 0
    del buf
    torch.cuda.empty_cache()


def test_stride_beyond_32_bits(rope):
    """A Q token stride of 2^32 + 256 elements (two tokens 8 GiB apart in bf16): the
    row-group kernel takes 32-bit strides, so the library runs the token kernel; the
    result matches the oracle (positions shifted by an offset so neither is the
    identity) and the memory between the rows stays untouched."""
    D, stride = 128, (1 << 32) + 256
    print("[parity] token stride beyond 32 bits", flush=True)
    buf = torch.zeros(stride + D, dtype=torch.bfloat16, device=DEV)
    vals = workloads.make_tensor((2, 2, D), 9400, "bf16", device=DEV)
    q = buf.as_strided((2, 1, D), (stride, D, 1))
    q.copy_(vals[:, :1])
    k = vals[:, 1:].clone()
    cu_h = np.array([0, 2], dtype=np.int32)
    off_h = np.array([1000], dtype=np.int32)
    rope.qk_apply_ex_(q, k, 1e6, 1, cu_seqlens=torch.from_numpy(cu_h).to(DEV),
                      seq_offsets=torch.from_numpy(off_h).to(DEV))
    torch.cuda.synchronize()
    touched = np.ones(2, dtype=bool)
    for what, x0, got in (("q", vals[:, :1], q), ("k", vals[:, 1:], k)):
        x = bits(x0)
        ref = oracle.rope(x, cu_h, 1e6, 1, "bf16", seq_offsets=off_h)
        assert_parity("bf16", bits(got), ref, x, touched, f"stride32:{what}")
    assert torch.count_nonzero(buf[D:1 << 20]).item() == 0
    assert torch.count_nonzero(buf[stride - (1 << 20):stride]).item() == 0
    del buf
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- cos/sin tables

@pytest.mark.parametrize("name", ["qwen3_4b_packed", "qwen3_8b_padded"])
def test_table_equals_theta_path(rope, name):
    """Tables written by the library's cos/sin export (bit-exact with the oracle's)
    make the table path bit-identical to the theta path: the row-group kernel on the
    packed batch, the token kernel on the padded layout; forward and backward."""
    w = workloads.get(name)
    print(f"[table] {name} theta-table identity", flush=True)
    host = make_host(w)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = None if w.seqused is None else torch.from_numpy(w.seqused).to(DEV)
    rows = int(max(w.lengths))
    ct, st = rope.cos_sin_table(rows, w.D, w.theta, DEV)
    a = {what: t.to(DEV) for what, t in host.items()}
    b = {what: t.to(DEV) for what, t in host.items()}
    rope.qk_fwd_(a["q"], a["k"], cu, w.theta, seqused=su)
    rope.qk_bwd_(a["dq"], a["dk"], cu, w.theta, seqused=su)
    rope.qk_apply_table_(b["q"], b["k"], ct, st, 1, cu_seqlens=cu, seqused=su)
    rope.qk_apply_table_(b["dq"], b["dk"], ct, st, -1, cu_seqlens=cu, seqused=su)
    torch.cuda.synchronize()
    for what in a:
        wd = _word(a[what].dtype)
        assert torch.equal(a[what].view(wd), b[what].view(wd)), f"{name}:{what}"


TABLE_CASES = [
    ("f32", 16, 4, 2, 0, "cu"),
    ("bf16", 128, 8, 2, 0, "cu"),
    ("bf16", 128, 8, 2, 3, "cu"),
    ("f16", 64, 3, 5, 1, "offsets"),
    ("bf16", 80, 2, 1, 0, "ids"),       # 5 chunks per half row: the staged instance
    ("f32", 128, 5, 0, 0, "ids"),       # Q only
]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,tpw,mode", TABLE_CASES)
def test_table_random_vs_oracle(rope, dtype, D, Hq, Hkv, tpw, mode):
    """Arbitrary tables (uniform in [-1.5, 1.5], not cos/sin of anything) against the
    oracle's table rotation. The table has fewer rows than the longest sequence, so
    the tokens whose position has no row must come back untouched, as must the tokens
    outside every sequence."""
    print(f"[table] random {dtype} D={D} Hq={Hq} Hkv={Hkv} tpw={tpw} {mode}", flush=True)
    rng = np.random.default_rng(D * 7 + Hq)
    cu_np = np.array([0, 5, 22, 25, 64, 64, 300], dtype=np.int32)
    T, rows = 310, 150
    ct = rng.uniform(-1.5, 1.5, (rows, D // 2)).astype(np.float32)
    st = rng.uniform(-1.5, 1.5, (rows, D // 2)).astype(np.float32)
    so_np = np.array([3, 0, 140, 9, 0, 2], dtype=np.int32) if mode == "offsets" else None
    pid_np = rng.integers(-3, rows + 40, T).astype(np.int32) if mode == "ids" else None
    shapes = {"q": (T, Hq, D), "k": (T, Hkv, D), "dq": (T, Hq, D), "dk": (T, Hkv, D)}
    host = {what: workloads.make_tensor(shp, 900 + i, dtype)
            for i, (what, shp) in enumerate(shapes.items())}
    dev, flats = {}, {}
    for what, t in host.items():
        dev[what], flats[what], g = guarded(t)
    kw = dict(cu_seqlens=torch.from_numpy(cu_np).to(DEV), tokens_per_wave=tpw,
              seq_offsets=None if so_np is None else torch.from_numpy(so_np).to(DEV),
              position_ids=None if pid_np is None else torch.from_numpy(pid_np).to(DEV))
    if mode == "ids":
        kw["cu_seqlens"] = None
    ctd, std = torch.from_numpy(ct).to(DEV), torch.from_numpy(st).to(DEV)
    rope.qk_apply_table_(dev["q"], dev["k"], ctd, std, 1, **kw)
    rope.qk_apply_table_(dev["dq"], dev["dk"], ctd, std, -1, **kw)
    torch.cuda.synchronize()
    cu_o = None if mode == "ids" else cu_np
    pos, _ = oracle.positions(cu_np if cu_o is not None else None, T, None, seq_offsets=so_np,
                              position_ids=pid_np)
    touched = (pos >= 0) & (pos < rows)
    assert touched.any() and (~touched).any()
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        if host[what].numel() == 0:
            continue
        x = bits(host[what])
        ref = oracle.rope_table(x, cu_o, ct, st, direction, dtype, seq_offsets=so_np,
                                position_ids=pid_np)
        assert_parity(dtype, bits(dev[what]), ref, x, touched, f"table:{what}")
        assert guards_intact(flats[what], g), f"table:{what}: guard region written"


def test_table_on_fused_qkv_views(rope):
    """The table path on Q/K views into a fused QKV buffer [T, (Hq + 2 Hkv) D] gives the
    bits of the same call on contiguous copies, forward and backward; V is untouched."""
    w = workloads.get("qwen3_8b_packed")
    print("[table] fused QKV views", flush=True)
    T, Hq, Hkv, D = w.T, w.Hq, w.Hkv, w.D
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    ct, st = rope.cos_sin_table(int(max(w.lengths)), D, w.theta, DEV)
    for direction in (1, -1):
        buf = workloads.make_tensor((T, (Hq + 2 * Hkv) * D), 77 + direction, "bf16", device=DEV)
        v0 = buf[:, (Hq + Hkv) * D:].clone()
        q = buf[:, :Hq * D].view(T, Hq, D)
        k = buf[:, Hq * D:(Hq + Hkv) * D].view(T, Hkv, D)
        qc, kc = q.contiguous(), k.contiguous()
        rope.qk_apply_table_(qc, kc, ct, st, direction, cu_seqlens=cu)
        rope.qk_apply_table_(q, k, ct, st, direction, cu_seqlens=cu)
        torch.cuda.synchronize()
        assert torch.equal(q.contiguous().view(torch.int16), qc.view(torch.int16)), direction
        assert torch.equal(k.contiguous().view(torch.int16), kc.view(torch.int16)), direction
        assert torch.equal(buf[:, (Hq + Hkv) * D:].view(torch.int16), v0.view(torch.int16))


def test_grid_beyond_one_dispatch(rope):
    """2^26 + 4099 tokens of the smallest shape (one Q and one K head, D = 2): the
    row-group grid would exceed one dispatch (2^26 workgroups) and one wave per token
    would exceed the grid limit, so the library launches waves that walk two tokens
    each. Sampled rows (ends, sequence boundaries, around every 2^24 tokens, random)
    against the oracle, forward and backward."""
    T = (1 << 26) + 4099
    print(f"[parity] T={T} beyond one dispatch", flush=True)
    cu_np = np.array([0, 1000, 5_000_000, 40_000_003, T - 7, T], dtype=np.int32)
    cu = torch.from_numpy(cu_np).to(DEV)
    theta = 1e4
    host = {what: workloads.make_tensor((T, 1, 2), 5100 + i, "bf16", device=DEV, chunk_rows=1 << 22)
            for i, what in enumerate(("q", "k", "dq", "dk"))}
    rng = np.random.default_rng(5150)
    marks = np.concatenate([np.arange(m - 3, m + 3) for m in (1 << 24, 2 << 24, 3 << 24, 1 << 26)]
                           + [np.arange(c - 2, c + 2) for c in cu_np[1:-1]])
    tokens = np.unique(np.concatenate([np.arange(0, 64), np.arange(T - 64, T), marks,
                                       rng.integers(0, T, 4096)]))
    tokens = tokens[(tokens >= 0) & (tokens < T)]
    tok_dev = torch.from_numpy(tokens).to(DEV)
    before = {what: bits(t.index_select(0, tok_dev)) for what, t in host.items()}
    rope.qk_fwd_(host["q"], host["k"], cu, theta)
    rope.qk_bwd_(host["dq"], host["dk"], cu, theta)
    torch.cuda.synchronize()
    touched = np.ones(tokens.size, dtype=bool)
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        got = bits(host[what].index_select(0, tok_dev))
        ref = oracle.rope_rows(before[what], tokens, cu_np, theta, direction, "bf16", None,
                               NTHREADS)
        assert_parity("bf16", got, ref, before[what], touched, f"big-grid:{what}")
    del host
    torch.cuda.empty_cache()


def test_concurrent_streams(rope):
    """Calls on different streams are independent: two batches rotated concurrently on
    two streams (default priority) give the bits of the same calls made one after the
    other on the default stream."""
    print("[parity] two streams", flush=True)
    work = []
    for name in ("qwen3_8b_packed", "qwen3_4b_packed"):
        w = workloads.get(name)
        cu = torch.from_numpy(w.cu_seqlens).to(DEV)
        q = workloads.make_tensor(w.shape("q"), w.seed("q"), w.dtype, device=DEV)
        k = workloads.make_tensor(w.shape("k"), w.seed("k"), w.dtype, device=DEV)
        work.append((w, cu, q, k))
    ref = []
    for w, cu, q, k in work:
        qr, kr = q.clone(), k.clone()
        rope.qk_fwd_(qr, kr, cu, w.theta)
        rope.qk_bwd_(qr, kr, cu, w.theta)
        rope.qk_fwd_(qr, kr, cu, w.theta)
        ref.append((qr, kr))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [(q.clone(), k.clone()) for _, _, q, k in work]
    torch.cuda.synchronize()
    for it in range(3):  # forward, backward, forward, interleaved across the streams
        for (w, cu, _q, _k), (qg, kg), st in zip(work, got, streams):
            with torch.cuda.stream(st):
                if it == 1:
                    rope.qk_bwd_(qg, kg, cu, w.theta)
                else:
                    rope.qk_fwd_(qg, kg, cu, w.theta)
    torch.cuda.synchronize()
    for (qr, kr), (qg, kg) in zip(ref, got):
        assert torch.equal(qg.view(torch.int16), qr.view(torch.int16))
        assert torch.equal(kg.view(torch.int16), kr.view(torch.int16))


# ---------------------------------------------------------------- compact padded launches

def _used(cu_np, su_np):
    lens = np.diff(np.asarray(cu_np, dtype=np.int64))
    used = lens if su_np is None else np.minimum(np.asarray(su_np, dtype=np.int64), lens)
    return np.maximum(used, 0)


def _cu_valid(cu_np, su_np):
    return np.concatenate([[0], np.cumsum(_used(cu_np, su_np))]).astype(np.int32)


def _compact_seqused(cu_np, su_np, cv_np, valid):
    """Per sequence, the tokens a compact launch rotates for a non-decreasing cu_valid
    (matching or not) and count `valid`: workgroup index v lands in sequence s for
    cu_valid[s] <= v < cu_valid[s+1], at position v - cu_valid[s], so s rotates its
    first min(cu_valid[s+1], valid) - cu_valid[s] positions, at most its used count."""
    cv = np.asarray(cv_np, dtype=np.int64)
    eff = np.minimum(cv[1:], valid) - cv[:-1]
    return np.clip(eff, 0, _used(cu_np, su_np)).astype(np.int32)


def run_compact(rope, name, host, cu_np, su_np, cv_np, valid, theta, dtype, seq_offsets=None,
                pos_scale=1.0, index_mode=0, expect_seqused=None):
    """Forward on (q, k) and backward on (dq, dk) through rope_qk_apply_padded, against
    the oracle with `expect_seqused` (default: su_np) as the rotated prefix of each
    sequence; untouched rows and guard regions bit for bit."""
    print(f"[parity] compact {name} T={host['q'].shape[0]} {dtype} valid={valid}", flush=True)
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).to(DEV)
    su = None if su_np is None else torch.from_numpy(np.asarray(su_np, dtype=np.int32)).to(DEV)
    cv = torch.from_numpy(np.asarray(cv_np, dtype=np.int32)).to(DEV)
    so = None if seq_offsets is None else \
        torch.from_numpy(np.asarray(seq_offsets, dtype=np.int32)).to(DEV)
    dev, flats = {}, {}
    for what, t in host.items():
        dev[what], flats[what], g = guarded(t)
    for a, b, direction in (("q", "k", 1), ("dq", "dk", -1)):
        rope.qk_apply_padded_(dev[a], dev[b], theta, direction, cu, su, cv, valid,
                              seq_offsets=so, pos_scale=pos_scale, index_mode=index_mode)
    torch.cuda.synchronize()
    want_su = su_np if expect_seqused is None else expect_seqused
    T = host["q"].shape[0]
    pos, _ = oracle.positions(cu_np, T, want_su, seq_offsets)
    touched = pos >= 0
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        x = bits(host[what])
        ref = oracle.rope(x, cu_np, theta, direction, dtype, want_su, NTHREADS,
                          seq_offsets=seq_offsets, pos_scale=pos_scale)
        assert_parity(dtype, bits(dev[what]), ref, x, touched, f"compact {name}:{what}")
        assert guards_intact(flats[what], g), f"compact {name}:{what}: guard region written"
    return {what: bits(t) for what, t in dev.items()}


def test_padded_compact_workload(rope):
    """The Qwen3-8B batch padded to 8 x 2048 rows through the compact launch, with
    cu_valid from the library's prefix kernel: every element against the oracle,
    padded rows untouched, and bit for bit the seqused launch's result."""
    w = workloads.get("qwen3_8b_padded")
    host = make_host(w)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = torch.from_numpy(w.seqused).to(DEV)
    cv_dev = rope.valid_prefix(cu, su)
    cv = _cu_valid(w.cu_seqlens, w.seqused)
    assert np.array_equal(cv_dev.cpu().numpy(), cv)
    got = run_compact(rope, w.name, host, w.cu_seqlens, w.seqused, cv, int(cv[-1]), w.theta,
                      w.dtype)
    ref = run_and_check(rope, w.name, host, w.cu_seqlens, w.seqused, w.theta, w.dtype)
    for what in ("q", "k", "dq", "dk"):
        assert np.array_equal(got[what], ref[what]), what


def _ragged_padded(seed, B, S, Hq, Hkv, D, dtype, tail=0):
    """B sequences padded to S rows each (plus `tail` rows after the last), with an
    empty sequence, seqused beyond the length, a negative seqused and a zero one."""
    rng = np.random.default_rng(seed)
    cu = (np.arange(B + 1, dtype=np.int64) * S).astype(np.int32)
    su = rng.integers(1, S + 1, size=B).astype(np.int32)
    su[1], su[2], su[3] = S + 50, -3, 0
    cu[B] = cu[B] - 7                    # the last sequence is 7 rows short
    cu[5] = cu[4]                        # sequence 4 is empty
    T = B * S + tail
    host = {what: workloads.make_tensor((T, Hq if what in ("q", "dq") else Hkv, D), seed + i,
                                        dtype) for i, what in enumerate(("q", "k", "dq", "dk"))}
    return host, cu, su


COMPACT_EDGE = [
    # name, dtype, D, Hq, Hkv, extra
    ("bf16_D128", "bf16", 128, 4, 2, {}),
    ("f32_D64", "f32", 64, 3, 1, {}),
    ("f16_D128_offsets", "f16", 128, 2, 2, {"offsets": True}),
    ("bf16_pos_scale", "bf16", 128, 4, 2, {"pos_scale": 4.0}),
    ("bf16_int64", "bf16", 128, 4, 2, {"index_mode": 2}),
    ("bf16_no_seqused", "bf16", 128, 4, 2, {"no_seqused": True}),
    ("bf16_D80_staged", "bf16", 80, 4, 2, {}),       # nc = 5: the staged row-group instance
    ("bf16_D512_steps", "bf16", 512, 5, 3, {}),      # two row steps per workgroup
    ("bf16_D192_staged_steps", "bf16", 192, 5, 3, {}),  # staged, two steps
    ("bf16_D100_fallback", "bf16", 100, 4, 2, {}),   # 4-byte chunks, nc = 25: the seqused launch
    ("bf16_valid_short", "bf16", 128, 4, 2, {"valid_delta": -100}),
    ("bf16_cv_wide", "bf16", 128, 4, 2, {"cv_gap": 9}),
    ("bf16_cv_narrow", "bf16", 128, 4, 2, {"cv_gap": -9}),
]


@pytest.mark.parametrize("case", COMPACT_EDGE, ids=[c[0] for c in COMPACT_EDGE])
def test_padded_compact_edges(rope, case):
    """Ragged padded batches through the compact launch against the oracle: empty
    sequences, seqused past the length, negative and zero seqused, a token tail,
    per-sequence offsets (some shifting positions out of range), position scaling,
    forced 64-bit offsets, no seqused, a staged head size, one with two row steps per
    workgroup, one that falls back to the seqused launch, and cu_valid / counts that do
    not match the layout (fewer tokens rotated, never wrong ones)."""
    name, dtype, D, Hq, Hkv, extra = case
    B, S = 12, 96
    host, cu, su = _ragged_padded(7100 + len(name), B, S, Hq, Hkv, D, dtype, tail=5)
    if extra.get("no_seqused"):
        su = None
    offsets = None
    if extra.get("offsets"):
        offsets = np.full(B, 1000, dtype=np.int32)
        offsets[0], offsets[6] = -40, 2**31 - 60   # some positions leave [0, 2^31)
    cv = _cu_valid(cu, su)
    valid = int(cv[-1])
    expect = None
    if "valid_delta" in extra:
        valid += extra["valid_delta"]
        expect = _compact_seqused(cu, su, cv, valid)
    if "cv_gap" in extra:
        gaps = np.diff(cv.astype(np.int64)) + extra["cv_gap"]
        cv = np.concatenate([[0], np.cumsum(np.maximum(gaps, 0))]).astype(np.int32)
        valid = min(int(cv[-1]), host["q"].shape[0])
        expect = _compact_seqused(cu, su, cv, valid)
    run_compact(rope, name, host, cu, su, cv, valid, 1e4, dtype, seq_offsets=offsets,
                pos_scale=extra.get("pos_scale", 1.0), index_mode=extra.get("index_mode", 0),
                expect_seqused=expect)


def test_padded_compact_long_context(rope):
    """A padded layout that needs 64-bit offsets by itself: 4 sequences padded to
    131072 rows each (524288 rows, 32 + 8 heads, bf16), 54-97% of each row block
    used, through the compact launch forward and backward (its 429076 rotated tokens
    issued as 7 launches): sampled rows (sequence ends, both sides of every used /
    padded boundary and of every launch boundary, random rows) against the oracle,
    padded rows untouched."""
    import bench
    S, B, Hq, Hkv, D = 131072, 4, 32, 8, 128
    T = S * B
    assert T * (Hq + Hkv) * D >= 1 << 31
    print("[parity] compact padded, 64-bit offsets", flush=True)
    cu_h = (np.arange(B + 1, dtype=np.int64) * S).astype(np.int32)
    su_h = np.array([127000, 71003, 131072, 100001], dtype=np.int32)
    cu, su = torch.from_numpy(cu_h).to(DEV), torch.from_numpy(su_h).to(DEV)
    cv = rope.valid_prefix(cu, su)
    valid = int(su_h.sum())
    dev = {what: workloads.make_tensor((T, Hq if what in ("q", "dq") else Hkv, D), 9500 + i,
                                       "bf16", device=DEV, chunk_rows=65536)
           for i, what in enumerate(("q", "k", "dq", "dk"))}
    rng = np.random.default_rng(9550)
    marks = [np.arange(c - 3, c + 3) for c in cu_h[1:-1]]
    marks += [np.arange(a + u - 3, a + u + 3) for a, u in zip(cu_h[:-1], su_h)]
    # launch boundaries, from rotated-token index to row
    wv = workloads.Workload("c", 0, valid, Hq, Hkv, D, "bf16", 1e6,
                            np.array([0, valid], dtype=np.int32))
    vb = np.cumsum(bench.group_pieces(valid, wv))[:-1]
    assert len(vb) == 6
    cv_h = np.concatenate([[0], np.cumsum(su_h.astype(np.int64))])
    s_of = np.searchsorted(cv_h, vb, side="right") - 1
    marks += [np.arange(r - 4, r + 4) for r in cu_h[s_of] + (vb - cv_h[s_of])]
    tokens = np.unique(np.concatenate([np.arange(0, 32), np.arange(T - 32, T), *marks,
                                       rng.integers(0, T, 4096)]))
    tokens = tokens[(tokens >= 0) & (tokens < T)]
    tok_dev = torch.from_numpy(tokens).to(DEV)
    before = {what: bits(t.index_select(0, tok_dev)) for what, t in dev.items()}
    rope.qk_apply_padded_(dev["q"], dev["k"], 1e6, 1, cu, su, cv, valid)
    rope.qk_apply_padded_(dev["dq"], dev["dk"], 1e6, -1, cu, su, cv, valid)
    torch.cuda.synchronize()
    pos, _ = oracle.positions(cu_h, T, su_h)
    touched = pos[tokens] >= 0
    assert touched.any() and (~touched).any()
    for what, direction in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        got = bits(dev[what].index_select(0, tok_dev))
        ref = oracle.rope_rows(before[what], tokens, cu_h, 1e6, direction, "bf16", su_h,
                               NTHREADS)
        assert_parity("bf16", got, ref, before[what], touched, f"compact-long:{what}")
    del dev
    torch.cuda.empty_cache()


def test_padded_compact_qkv_views(rope):
    """The compact launch on Q and K as views into fused QKV outputs of a padded batch:
    bit for bit the seqused launch on the same views, V and padded rows untouched."""
    w = workloads.get("qwen3_8b_padded")
    Hq, Hkv, D = w.Hq, w.Hkv, w.D
    print("[parity] compact on fused qkv views", flush=True)
    qkv0 = workloads.make_tensor((w.T, (Hq + 2 * Hkv) * D), 9300, "bf16", device=DEV)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = torch.from_numpy(w.seqused).to(DEV)
    cv = rope.valid_prefix(cu, su)
    valid = int(_cu_valid(w.cu_seqlens, w.seqused)[-1])
    a, b = qkv0.clone(), qkv0.clone()
    for direction in (1, -1):
        qa, ka, _ = _qkv_views(a, Hq, Hkv, D)
        qb, kb, _ = _qkv_views(b, Hq, Hkv, D)
        rope.qk_apply_padded_(qa, ka, w.theta, direction, cu, su, cv, valid)
        rope.qk_apply_ex_(qb, kb, w.theta, direction, cu_seqlens=cu, seqused=su)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    pos, _ = oracle.positions(w.cu_seqlens, w.T, w.seqused)
    pad = torch.from_numpy(pos < 0).to(DEV)
    assert torch.equal(a[pad].view(torch.int16), qkv0[pad].view(torch.int16))
    _, _, v = _qkv_views(a, Hq, Hkv, D)
    _, _, v0 = _qkv_views(qkv0, Hq, Hkv, D)
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16))


@pytest.mark.parametrize("B", [0, 1, 7, 255, 256, 257, 1000, 5000])
def test_valid_prefix(rope, B):
    """rope_valid_prefix against the running sum of min(seqused, length) clamped at 0,
    with and without seqused, over several scan steps: bit-exact."""
    print(f"[parity] valid_prefix B={B}", flush=True)
    rng = np.random.default_rng(7300 + B)
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.1] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    su = rng.integers(-5, 3200, size=B).astype(np.int32)
    for seqused in (su, None):
        got = rope.valid_prefix(torch.from_numpy(cu).to(DEV),
                                None if seqused is None else torch.from_numpy(seqused).to(DEV))
        assert np.array_equal(got.cpu().numpy(), _cu_valid(cu, seqused))


def test_valid_prefix_saturates(rope):
    """Counts beyond INT32_MAX saturate; a decreasing cu_seqlens contributes 0."""
    big = 2**31 - 1
    cu = torch.tensor([-big, big, -big, big], dtype=torch.int32, device=DEV)
    su = torch.full((3,), big, dtype=torch.int32, device=DEV)
    got = rope.valid_prefix(cu, su).cpu().numpy()
    assert got.tolist() == [0, big, big, big]
