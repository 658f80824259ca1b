"""GPU tests of the autograd entry points (packed_varlen_rotary_rope_amd.functional)
and of HIP-graph capture and replay of the kernels.

Autograd: gradients through rope_qk / glu / glu_fused equal, bit for bit, the
direct backward launches on the same upstream gradients, and agree with the
oracle. Graphs: a captured forward+backward, replayed several times with eager
work and synchronizations in between, gives every time the bits of the eager
launches on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import glu as glu_oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_rotary_rope_amd as m
    import packed_varlen_rotary_rope_amd.functional as F
    return m, F


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("inplace_backward", [False, True])
def test_rope_autograd_matches_direct_launches(lib, inplace_backward):
    """loss = <rope(q), wq> + <rope(k), wk>: dL/dq is the backward rotation of wq,
    so q's gradient must equal qk_bwd_ applied to wq (bit for bit), and the oracle's
    backward of wq (1 bf16 ulp)."""
    rope, F = lib
    w = workloads.get("qwen3_8b_packed")
    print(f"[autograd] rope_qk inplace_backward={inplace_backward}", flush=True)
    q0 = workloads.make_tensor(w.shape("q"), 31, "bf16", device=DEV).requires_grad_()
    k0 = workloads.make_tensor(w.shape("k"), 32, "bf16", device=DEV).requires_grad_()
    wq = workloads.make_tensor(w.shape("q"), 33, "bf16", device=DEV)
    wk = workloads.make_tensor(w.shape("k"), 34, "bf16", device=DEV)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    q, k = q0 * 1, k0 * 1  # non-leaf inputs, as projection outputs are
    qr, kr = F.rope_qk(q, k, cu, w.theta, inplace_backward=inplace_backward)
    ((qr.float() * wq.float()).sum() + (kr.float() * wk.float()).sum()).backward()
    # forward result equals the direct launch
    qd, kd = q0.detach().clone(), k0.detach().clone()
    rope.qk_fwd_(qd, kd, cu, w.theta)
    gq, gk = wq.clone(), wk.clone()
    rope.qk_bwd_(gq, gk, cu, w.theta)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(qr), bits16(qd)) and np.array_equal(bits16(kr), bits16(kd))
    assert np.array_equal(bits16(q0.grad), bits16(gq))
    assert np.array_equal(bits16(k0.grad), bits16(gk))
    ref = oracle.rope(bits16(wq), w.cu_seqlens, w.theta, -1, "bf16", nthreads=8)
    got = bits16(q0.grad).astype(np.int64)
    want = oracle.round_bf16(ref).astype(np.int64)

    def ordered(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b)

    assert int(np.abs(ordered(got) - ordered(want)).max()) <= 1


def test_rope_autograd_compact_padded(lib):
    """The padded Qwen3-8B batch through rope_qk with cu_valid / valid_tokens (the
    compact launch, both passes): output and gradients bit for bit those of the
    seqused launch, padded rows and their gradients passed through unchanged."""
    rope, F = lib
    w = workloads.get("qwen3_8b_padded")
    print("[autograd] rope_qk compact padded", flush=True)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    su = torch.from_numpy(w.seqused).to(DEV)
    cv = rope.valid_prefix(cu, su)
    wq = workloads.make_tensor(w.shape("q"), 43, "bf16", device=DEV)
    wk = workloads.make_tensor(w.shape("k"), 44, "bf16", device=DEV)
    res = []
    for compact in (True, False):
        q0 = workloads.make_tensor(w.shape("q"), 41, "bf16", device=DEV).requires_grad_()
        k0 = workloads.make_tensor(w.shape("k"), 42, "bf16", device=DEV).requires_grad_()
        kw = dict(cu_valid=cv, valid_tokens=w.valid_tokens) if compact else {}
        qr, kr = F.rope_qk(q0 * 1, k0 * 1, cu, w.theta, seqused=su, **kw)
        ((qr.float() * wq.float()).sum() + (kr.float() * wk.float()).sum()).backward()
        torch.cuda.synchronize()
        res.append([bits16(t) for t in (qr, kr, q0.grad, k0.grad)])
    for a, b in zip(*res):
        assert np.array_equal(a, b)
    pos, _ = oracle.positions(w.cu_seqlens, w.T, w.seqused)
    pad = pos < 0
    assert np.array_equal(res[0][2][pad], bits16(wq)[pad])  # gradient of a padded row: wq


@pytest.mark.parametrize("inplace_backward", [False, True])
def test_rope_table_autograd_matches_theta_path(lib, inplace_backward):
    """rope_qk_table with the library's own cos/sin tables gives the outputs and the
    input gradients of rope_qk, bit for bit; the tables get no gradient."""
    rope, F = lib
    w = workloads.get("qwen3_8b_packed")
    print(f"[autograd] rope_qk_table inplace_backward={inplace_backward}", flush=True)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    ct, st = rope.cos_sin_table(int(max(w.lengths)), w.D, w.theta, DEV)
    wq = workloads.make_tensor(w.shape("q"), 43, "bf16", device=DEV)
    wk = workloads.make_tensor(w.shape("k"), 44, "bf16", device=DEV)
    outs = []
    for use_table in (False, True):
        q0 = workloads.make_tensor(w.shape("q"), 41, "bf16", device=DEV).requires_grad_()
        k0 = workloads.make_tensor(w.shape("k"), 42, "bf16", device=DEV).requires_grad_()
        q, k = q0 * 1, k0 * 1
        if use_table:
            qr, kr = F.rope_qk_table(q, k, ct, st, cu, inplace_backward=inplace_backward)
        else:
            qr, kr = F.rope_qk(q, k, cu, w.theta, inplace_backward=inplace_backward)
        ((qr.float() * wq.float()).sum() + (kr.float() * wk.float()).sum()).backward()
        torch.cuda.synchronize()
        outs.append([bits16(t) for t in (qr, kr, q0.grad, k0.grad)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert ct.grad is None and st.grad is None


def test_rope_autograd_shared_gradient_is_not_clobbered(lib):
    """out = rope(q) + x: autograd hands the same gradient tensor to both operands;
    the default backward must leave x's gradient unrotated."""
    rope, F = lib
    T, H, D = 64, 2, 32
    cu = torch.tensor([0, 40, 64], dtype=torch.int32, device=DEV)
    q0 = torch.randn(T, H, D, device=DEV, requires_grad=True)
    x = torch.randn(T, H, D, device=DEV, requires_grad=True)
    k = torch.zeros(T, 0, D, device=DEV)
    qr, _ = F.rope_qk(q0 * 1, k, cu, 1e4)
    upstream = torch.randn(T, H, D, device=DEV)
    (qr + x).backward(upstream)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, upstream)
    expect = upstream.clone()
    rope.qk_bwd_(expect, torch.zeros(T, 0, D, device=DEV), cu, 1e4)
    assert torch.equal(q0.grad, expect)


def _projection(T, n_in, n_out, seed):
    """fp32 input and weight (the products and their backward stay in fp32); the
    projection output is cast to bf16 by the caller."""
    x = workloads.make_tensor((T, n_in), seed, "f32", device=DEV).requires_grad_()
    w = (workloads.make_tensor((n_in, n_out), seed + 1, "f32", device=DEV) * 0.05).contiguous()
    return x, w


def test_rope_qk_on_projection_views(lib):
    """The usual model code: q = (x @ Wq).view(T, Hq, D), k = (x @ Wk).view(T, Hkv, D),
    views that require grad. rope_qk returns the rotation of their values, and the
    gradient reaching each projection output is the backward rotation of the upstream
    gradient, bit for bit against direct launches."""
    rope, F = lib
    w = workloads.get("qwen3_8b_packed")
    print("[autograd] rope_qk on projection views", flush=True)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    x, wq = _projection(w.T, 256, w.Hq * w.D, 51)
    wk = (workloads.make_tensor((256, w.Hkv * w.D), 53, "f32", device=DEV) * 0.05).contiguous()
    pq, pk = (x @ wq).to(torch.bfloat16), (x @ wk).to(torch.bfloat16)
    grads = {}
    pq.register_hook(lambda g: grads.__setitem__("q", g.detach().clone()))
    pk.register_hook(lambda g: grads.__setitem__("k", g.detach().clone()))
    q, k = pq.view(w.T, w.Hq, w.D), pk.view(w.T, w.Hkv, w.D)
    qr, kr = F.rope_qk(q, k, cu, w.theta)
    uq = workloads.make_tensor(w.shape("q"), 55, "bf16", device=DEV)
    uk = workloads.make_tensor(w.shape("k"), 56, "bf16", device=DEV)
    ((qr.float() * uq.float()).sum() + (kr.float() * uk.float()).sum()).backward()
    qd = pq.detach().view(w.T, w.Hq, w.D).clone()
    kd = pk.detach().view(w.T, w.Hkv, w.D).clone()
    rope.qk_fwd_(qd, kd, cu, w.theta)
    gq, gk = uq.clone(), uk.clone()
    rope.qk_bwd_(gq, gk, cu, w.theta)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(qr), bits16(qd)) and np.array_equal(bits16(kr), bits16(kd))
    assert np.array_equal(bits16(grads["q"].view(w.shape("q"))), bits16(gq))
    assert np.array_equal(bits16(grads["k"].view(w.shape("k"))), bits16(gk))
    assert x.grad is not None and bool(torch.isfinite(x.grad.float()).all())


@pytest.mark.parametrize("shape3,inplace_backward", [(False, False), (True, False), (True, True)])
def test_rope_qkv_fused_projection(lib, shape3, inplace_backward):
    """rope_qkv on a fused projection output (x @ Wqkv, viewed as [T, H*D] or
    [T, Hq+2Hkv, D]): Q and K rotated in place in one launch, V untouched; the
    gradient into the projection is [bwd(dQ), bwd(dK), dV], bit for bit."""
    rope, F = lib
    w = workloads.get("qwen3_8b_packed")
    print(f"[autograd] rope_qkv shape3={shape3} inplace_backward={inplace_backward}", flush=True)
    H = w.Hq + 2 * w.Hkv
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    x, wqkv = _projection(w.T, 256, H * w.D, 61)
    proj = (x @ wqkv).to(torch.bfloat16)
    got = {}
    proj.register_hook(lambda g: got.__setitem__("g", g.detach().clone()))
    before = proj.detach().clone()
    qkv = proj.view(w.T, H, w.D) if shape3 else proj.view(w.T, -1)
    out = F.rope_qkv(qkv, w.Hq, w.Hkv, cu, w.theta, inplace_backward=inplace_backward)
    assert out.data_ptr() == proj.data_ptr()
    up = workloads.make_tensor((w.T, H * w.D), 63, "bf16", device=DEV)
    (out.float() * up.view(out.shape).float()).sum().backward()
    nq, nk = w.Hq * w.D, w.Hkv * w.D
    qd = before[:, :nq].contiguous().view(w.shape("q"))
    kd = before[:, nq:nq + nk].contiguous().view(w.shape("k"))
    rope.qk_fwd_(qd, kd, cu, w.theta)
    gq = up[:, :nq].contiguous().view(w.shape("q"))
    gk = up[:, nq:nq + nk].contiguous().view(w.shape("k"))
    rope.qk_bwd_(gq, gk, cu, w.theta)
    torch.cuda.synchronize()
    o = out.detach().reshape(w.T, -1)
    assert np.array_equal(bits16(o[:, :nq]), bits16(qd.view(w.T, -1)))
    assert np.array_equal(bits16(o[:, nq:nq + nk]), bits16(kd.view(w.T, -1)))
    assert np.array_equal(bits16(o[:, nq + nk:]), bits16(before[:, nq + nk:]))
    g = got["g"]
    assert np.array_equal(bits16(g[:, :nq]), bits16(gq.view(w.T, -1)))
    assert np.array_equal(bits16(g[:, nq:nq + nk]), bits16(gk.view(w.T, -1)))
    assert np.array_equal(bits16(g[:, nq + nk:]), bits16(up[:, nq + nk:]))


@pytest.mark.parametrize("kind", ["swiglu", "geglu", "geglu_tanh"])
def test_glu_autograd(lib, kind):
    """glu and glu_fused: forward and gradients equal the direct launches bit for
    bit, and the fused gradient is one buffer whose halves are de and dg."""
    rope, F = lib
    rows, cols = 513, 1024
    print(f"[autograd] glu {kind}", flush=True)
    gu = workloads.make_tensor((rows, 2 * cols), 41, "bf16", device=DEV).requires_grad_()
    e0 = workloads.make_tensor((rows, cols), 42, "bf16", device=DEV).requires_grad_()
    g0 = workloads.make_tensor((rows, cols), 43, "bf16", device=DEV).requires_grad_()
    dh = workloads.make_tensor((rows, cols), 44, "bf16", device=DEV)
    h = F.glu(kind, e0, g0)
    h.backward(dh)
    hf = F.glu_fused(kind, gu)
    hf.backward(dh)
    h_ref = rope.glu_fwd(kind, e0.detach(), g0.detach())
    de_ref, dg_ref = rope.glu_bwd(kind, dh, e0.detach(), g0.detach())
    e1, g1 = gu.detach()[:, :cols], gu.detach()[:, cols:]
    hf_ref = rope.glu_fwd(kind, e1, g1)
    def1, dgf1 = rope.glu_bwd(kind, dh, e1, g1)
    torch.cuda.synchronize()
    for a, b in ((h, h_ref), (e0.grad, de_ref), (g0.grad, dg_ref), (hf, hf_ref),
                 (gu.grad[:, :cols], def1), (gu.grad[:, cols:], dgf1)):
        assert np.array_equal(bits16(a), bits16(b))
    # and the oracle agrees with the autograd gradient of e (1 bf16 ulp)
    ref_de, _ = glu_oracle.bwd(kind, bits16(dh), bits16(e0), bits16(g0), "bf16", 8)
    want = glu_oracle.round_to("bf16", ref_de).astype(np.int64)
    got = bits16(e0.grad).astype(np.int64)

    def ordered(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b)

    assert int(np.abs(ordered(got) - ordered(want)).max()) <= 1


def test_graph_capture_replay(lib):
    """RoPE forward + backward, a compact padded forward (with its cu_valid made by
    the prefix kernel inside the graph), SwiGLU forward + backward, and two calls
    long enough to go out as several launches (a RoPE forward over 73000 tokens of
    64 + 8 heads: 3 launches; a SwiGLU forward over 65536 x 8192: 2 launches)
    captured in one HIP graph on static buffers; four replays, each after fresh
    inputs are copied in and with eager launches and synchronizations between
    replays, each equal bit for bit to eager launches on the same inputs."""
    rope, F = lib
    w = workloads.get("qwen3_4b_packed")
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    wp = workloads.get("qwen3_8b_padded")
    cu_p, su_p = torch.from_numpy(wp.cu_seqlens).to(DEV), torch.from_numpy(wp.seqused).to(DEV)
    cv = torch.full((cu_p.numel(),), -1, dtype=torch.int32, device=DEV)
    pq = torch.empty(wp.shape("q"), dtype=torch.bfloat16, device=DEV)
    pk = torch.empty(wp.shape("k"), dtype=torch.bfloat16, device=DEV)
    rows, cols = 2048, 4096
    static = {n: torch.empty(w.shape(n), dtype=torch.bfloat16, device=DEV)
              for n in ("q", "k", "dq", "dk")}
    ge, gg, gdh = (torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    gh = torch.empty_like(ge)
    gde, gdg = torch.empty_like(ge), torch.empty_like(ge)
    LT, LHq, LHkv = 73000, 64, 8  # 657000 workgroups: 3 launches
    lcu = torch.tensor([0, 20000, 24336, 50001, LT], dtype=torch.int32, device=DEV)
    lq = torch.empty((LT, LHq, 128), dtype=torch.bfloat16, device=DEV)
    lk = torch.empty((LT, LHkv, 128), dtype=torch.bfloat16, device=DEV)
    Lr, Lc = 65536, 8192  # 65536 workgroups: 2 launches
    le, lg = (torch.empty((Lr, Lc), dtype=torch.bfloat16, device=DEV) for _ in range(2))
    lh = torch.empty_like(le)

    def body():
        rope.qk_fwd_(static["q"], static["k"], cu, w.theta)
        rope.qk_bwd_(static["dq"], static["dk"], cu, w.theta)
        rope.glu_fwd("swiglu", ge, gg, out=gh)
        rope.glu_bwd("swiglu", gdh, ge, gg, de=gde, dg=gdg)
        rope.valid_prefix(cu_p, su_p, out=cv)
        rope.qk_apply_padded_(pq, pk, wp.theta, 1, cu_p, su_p, cv, wp.valid_tokens)
        rope.qk_fwd_(lq, lk, lcu, 1e6)
        rope.glu_fwd("swiglu", le, lg, out=lh)

    # warm up on a side stream, as torch requires before capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for rep in range(4):
        print(f"[graph] replay {rep}", flush=True)
        inputs = {n: workloads.make_tensor(w.shape(n), 500 + 10 * rep + i, "bf16", device=DEV)
                  for i, n in enumerate(("q", "k", "dq", "dk"))}
        ins = [workloads.make_tensor((rows, cols), 600 + 10 * rep + i, "bf16", device=DEV)
               for i in range(3)]
        for n in static:
            static[n].copy_(inputs[n])
        for dst, src in zip((ge, gg, gdh), ins):
            dst.copy_(src)
        pin = [workloads.make_tensor(wp.shape(n), 700 + 10 * rep + i, "bf16", device=DEV)
               for i, n in enumerate(("q", "k"))]
        pq.copy_(pin[0])
        pk.copy_(pin[1])
        cv.fill_(-1)
        lin = [workloads.make_tensor(shape, 800 + 10 * rep + i, "bf16", device=DEV, chunk_rows=8192)
               for i, shape in enumerate(((LT, LHq, 128), (LT, LHkv, 128), (Lr, Lc), (Lr, Lc)))]
        for dst, src in zip((lq, lk, le, lg), lin):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        # eager reference on separate copies, with its own synchronizations
        eager = {n: t.clone() for n, t in inputs.items()}
        rope.qk_fwd_(eager["q"], eager["k"], cu, w.theta)
        rope.qk_bwd_(eager["dq"], eager["dk"], cu, w.theta)
        h = rope.glu_fwd("swiglu", ins[0], ins[1])
        de, dg = rope.glu_bwd("swiglu", ins[2], ins[0], ins[1])
        rope.qk_apply_ex_(pin[0], pin[1], wp.theta, 1, cu_seqlens=cu_p, seqused=su_p)
        rope.qk_fwd_(lin[0], lin[1], lcu, 1e6)
        lh_eager = rope.glu_fwd("swiglu", lin[2], lin[3])
        torch.cuda.synchronize()
        assert torch.equal(lq.view(torch.int16), lin[0].view(torch.int16)), rep
        assert torch.equal(lk.view(torch.int16), lin[1].view(torch.int16)), rep
        assert torch.equal(lh.view(torch.int16), lh_eager.view(torch.int16)), rep
        assert np.array_equal(bits16(pq), bits16(pin[0])) and np.array_equal(bits16(pk), bits16(pin[1]))
        assert cv.cpu().tolist() == rope.valid_prefix(cu_p, su_p).cpu().tolist()
        for n in static:
            assert np.array_equal(bits16(static[n]), bits16(eager[n])), (rep, n)
        for a, b in ((gh, h), (gde, de), (gdg, dg)):
            assert np.array_equal(bits16(a), bits16(b)), rep
