"""Host logic of the autograd layer (packed_varlen_rotary_rope_amd.functional) on the
CPU: the library call is replaced by a stand-in with the same in-place contract
(scale Q by 2 and K by 3 in either direction: a symmetric map, so its backward is
itself), which checks how rope_qk and rope_qkv wire their inputs, views and
gradients into autograd. The rotation itself is tested on the GPU."""
import pytest
import torch

import packed_varlen_rotary_rope_amd.functional as F

T, Hq, Hkv, D = 6, 4, 2, 8


@pytest.fixture
def stand_in(monkeypatch):
    calls = []

    def fake_apply(q, k, theta, direction, **kw):
        assert q.stride(-1) == 1 and k.stride(-1) == 1
        calls.append((q.data_ptr(), k.data_ptr(), direction))
        with torch.no_grad():
            q.mul_(2.0)
            k.mul_(3.0)
        return q, k

    monkeypatch.setattr(F, "qk_apply_ex_", fake_apply)
    return calls


def cu():
    return torch.tensor([0, 2, T], dtype=torch.int32)


def test_rope_qk_on_projection_views(stand_in):
    """q = (x @ Wq).view(...) and k likewise: views that require grad. rope_qk must
    work (on copies) and send the backward map of the upstream gradient to x."""
    torch.manual_seed(0)
    x = torch.randn(T, 16, dtype=torch.float64, requires_grad=True)
    wq, wk = torch.randn(16, Hq * D, dtype=torch.float64), torch.randn(16, Hkv * D,
                                                                         dtype=torch.float64)
    q, k = (x @ wq).view(T, Hq, D), (x @ wk).view(T, Hkv, D)
    qr, kr = F.rope_qk(q, k, cu(), 1e4)
    assert torch.equal(qr, 2 * (x @ wq).view(T, Hq, D)) and torch.equal(kr, 3 * (x @ wk).view(T, Hkv, D))
    gq, gk = torch.randn_like(qr), torch.randn_like(kr)
    ((qr * gq).sum() + (kr * gk).sum()).backward()
    want = (2 * gq).flatten(1) @ wq.T + (3 * gk).flatten(1) @ wk.T
    assert torch.allclose(x.grad, want, rtol=1e-12, atol=1e-12)
    assert [c[2] for c in stand_in] == [1, -1]


def test_rope_qk_non_view_stays_in_place(stand_in):
    x = torch.randn(T, Hq, D, requires_grad=True)
    q = x * 1
    k = torch.randn(T, Hkv, D, requires_grad=True) * 1
    qp = q.data_ptr()
    qr, _ = F.rope_qk(q, k, cu(), 1e4)
    assert qr.data_ptr() == qp and stand_in[0][0] == qp


@pytest.mark.parametrize("shape3", [False, True])
def test_rope_qkv_fused_view(stand_in, shape3):
    """rope_qkv on (x @ W).view(...): Q and K columns rotated in place in one call,
    V untouched, gradient [backward(dQ), backward(dK), dV] into the projection."""
    torch.manual_seed(1)
    x = torch.randn(T, 16, dtype=torch.float64, requires_grad=True)
    w = torch.randn(16, (Hq + 2 * Hkv) * D, dtype=torch.float64)
    proj = x @ w
    qkv = proj.view(T, Hq + 2 * Hkv, D) if shape3 else proj.view(T, -1)
    before = proj.detach().clone()
    out = F.rope_qkv(qkv, Hq, Hkv, cu(), 1e4)
    assert out.data_ptr() == proj.data_ptr() and len(stand_in) == 1
    flat = out.detach().reshape(T, -1)
    nq, nk = Hq * D, Hkv * D
    assert torch.equal(flat[:, :nq], 2 * before[:, :nq])
    assert torch.equal(flat[:, nq:nq + nk], 3 * before[:, nq:nq + nk])
    assert torch.equal(flat[:, nq + nk:], before[:, nq + nk:])
    g = torch.randn_like(out)
    (out * g).sum().backward()
    gf = g.reshape(T, -1)
    scale = torch.cat([torch.full((nq,), 2.0), torch.full((nk,), 3.0), torch.ones(nk)]).double()
    assert torch.allclose(x.grad, (gf * scale) @ w.T, rtol=1e-12, atol=1e-12)
    assert stand_in[1][2] == -1


def test_rope_qkv_rejects_bad_layouts():
    with pytest.raises(ValueError):
        F._qkv_split(torch.zeros(T, 7 * D + 1), Hq, Hkv)  # columns not a multiple of heads
    with pytest.raises(ValueError):
        F._qkv_split(torch.zeros(T, Hq + 2 * Hkv + 1, D), Hq, Hkv)
    with pytest.raises(ValueError):
        F._qkv_split(torch.zeros(D, Hq + 2 * Hkv, T).transpose(0, 2), Hq, Hkv)


def test_rope_qk_compact_padded_routing(monkeypatch):
    """With cu_valid and valid_tokens, forward and backward both take the compact padded
    entry point with the same metadata; position_ids or a missing count are refused."""
    calls = []

    def fake_padded(q, k, theta, direction, cu_seqlens, seqused, cu_valid, valid_tokens, **kw):
        calls.append((direction, cu_valid.data_ptr(), valid_tokens))
        with torch.no_grad():
            q.mul_(2.0)
            k.mul_(3.0)
        return q, k

    def no_ex(*a, **kw):
        raise AssertionError("the general entry point was called")

    monkeypatch.setattr(F, "qk_apply_padded_", fake_padded)
    monkeypatch.setattr(F, "qk_apply_ex_", no_ex)
    x = torch.randn(T, (Hq + Hkv) * D, requires_grad=True)
    q = (x[:, :Hq * D] * 1.0).reshape(T, Hq, D).contiguous()
    k = (x[:, Hq * D:] * 1.0).reshape(T, Hkv, D).contiguous()
    su = torch.tensor([1, 3], dtype=torch.int32)
    cv = torch.tensor([0, 1, 4], dtype=torch.int32)
    qr, kr = F.rope_qk(q, k, cu(), 1e4, seqused=su, cu_valid=cv, valid_tokens=4)
    (qr.sum() + kr.sum()).backward()
    assert calls == [(1, cv.data_ptr(), 4), (-1, cv.data_ptr(), 4)]
    assert torch.allclose(x.grad[:, :Hq * D], torch.full((T, Hq * D), 2.0))
    with pytest.raises(ValueError):
        F.rope_qk(q.detach(), k.detach(), cu(), 1e4, cu_valid=cv)  # no count
    with pytest.raises(ValueError):
        F.rope_qk(q.detach(), k.detach(), None, 1e4, position_ids=torch.zeros(T, dtype=torch.int32),
                  cu_valid=cv, valid_tokens=4)
