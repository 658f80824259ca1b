"""Autograd entry points over the C ABI: the packed-varlen QK rotary embedding
and the SwiGLU / GeGLU activations as differentiable torch functions.

Every pass is one launch of the library's kernels on the current stream (a long
pass: several, over consecutive ranges); this module only wires them into
torch.autograd (no arithmetic of its own).

    qkv = rope_qkv(qkv, Hq, Hkv, cu_seqlens, theta)  # fused QKV output, in place
    q, k = rope_qk(q, k, cu_seqlens, theta)        # returns q and k, rotated
    q, k = rope_qk(q, k, cu, theta, seqused=su,    # padded layout, launched over its
                   cu_valid=valid_prefix(cu, su), valid_tokens=n)  # n rotated tokens only
    q, k = rope_qk_table(q, k, cos_tab, sin_tab, cu_seqlens)  # cos/sin from tables
    h = glu("swiglu", e, g)                        # h = silu(e) * g
    h = glu_fused("geglu", gate_up)                # e, g = halves of gate_up

The RoPE functions rotate in place (their inputs are marked dirty), so the
inputs must not be leaf tensors that require grad -- in a model they are
projection outputs. rope_qkv takes the fused projection output [T, (Hq + 2 Hkv)
* D] (or [T, Hq + 2 Hkv, D]) and rotates its Q and K columns in one strided
launch, V untouched; it is one in-place output, which autograd accepts also when
the buffer is a view (e.g. ``(x @ W).view(...)``). rope_qk takes q and k as two
tensors: autograd cannot mark two outputs of one function dirty when an input is
a view of another tensor, so a q or k that is such a view and requires grad is
rotated on a contiguous copy (one extra read and write of it; rope_qkv avoids
that for fused projections). Either way use the returned tensors.

The backward applies the transposed rotation (sin negated, Unsloth, "Entrainement
des LLM 3 fois plus rapide...", fused QK RoPE section) to the incoming
gradients: in place on them when ``inplace_backward=True``, otherwise on a copy,
because autograd may hand the same gradient tensor to several consumers (an
addition passes its gradient to both operands), and rotating a shared tensor in
place would change the other consumer's gradient.
"""
from __future__ import annotations

import torch

from . import glu_bwd, glu_fwd, qk_apply_ex_, qk_apply_padded_, qk_apply_table_


def _rotate(q, k, theta, direction, cu, su, pid, so, pos_scale, cv, valid):
    """One launch: the compact padded launch when cu_valid is given, else the general one."""
    if cv is not None:
        qk_apply_padded_(q, k, theta, direction, cu, su, cv, valid, seq_offsets=so,
                         pos_scale=pos_scale)
    else:
        qk_apply_ex_(q, k, theta, direction, cu_seqlens=cu, seqused=su, seq_offsets=so,
                     position_ids=pid, pos_scale=pos_scale)


def _padded_args(position_ids, cu_valid, valid_tokens):
    if cu_valid is None:
        return None
    if position_ids is not None or valid_tokens is None:
        raise ValueError("cu_valid goes with cu_seqlens and valid_tokens, not position_ids")
    return int(valid_tokens)


class _RopeQK(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, cu_seqlens, theta, seqused, position_ids, seq_offsets, pos_scale,
                inplace_backward, cu_valid, valid_tokens):
        _rotate(q, k, theta, 1, cu_seqlens, seqused, position_ids, seq_offsets, pos_scale,
                cu_valid, valid_tokens)
        ctx.mark_dirty(q, k)
        ctx.save_for_backward(cu_seqlens, seqused, position_ids, seq_offsets, cu_valid)
        ctx.theta, ctx.pos_scale, ctx.inplace = theta, pos_scale, inplace_backward
        ctx.valid = valid_tokens
        return q, k

    @staticmethod
    def backward(ctx, dq, dk):
        # gradients that did not flow arrive as zeros (materialized by autograd)
        cu, su, pid, so, cv = ctx.saved_tensors
        if not (ctx.inplace and dq.is_contiguous()):
            dq = dq.clone(memory_format=torch.contiguous_format)
        if not (ctx.inplace and dk.is_contiguous()):
            dk = dk.clone(memory_format=torch.contiguous_format)
        _rotate(dq, dk, ctx.theta, -1, cu, su, pid, so, ctx.pos_scale, cv, ctx.valid)
        return dq, dk, None, None, None, None, None, None, None, None, None


def _own_storage(t: torch.Tensor) -> torch.Tensor:
    """t itself, or a contiguous copy when t is a view that requires grad (autograd
    refuses an in-place function with two outputs on such an input)."""
    if torch.is_grad_enabled() and t.requires_grad and t._is_view():
        return t.clone(memory_format=torch.contiguous_format)
    return t


def rope_qk(q: torch.Tensor, k: torch.Tensor, cu_seqlens=None, theta: float = 10000.0,
            seqused=None, position_ids=None, seq_offsets=None, pos_scale: float = 1.0,
            inplace_backward: bool = False, cu_valid=None, valid_tokens=None):
    """Differentiable RoPE of q [T, Hq, D] and k [T, Hkv, D] (views with contiguous
    heads, e.g. slices of a fused QKV output, are accepted), in place unless q or k
    is a view that requires grad (then on a copy of it; see the module docstring and
    rope_qkv). Positions come from cu_seqlens (with optional seqused / seq_offsets)
    or position_ids, as in ``qk_apply_ex_``; with ``cu_valid`` (from ``valid_prefix``)
    and ``valid_tokens``, a padded layout is launched over its rotated tokens only, as
    in ``qk_apply_padded_`` (same results). Returns (q, k), rotated."""
    valid = _padded_args(position_ids, cu_valid, valid_tokens)
    return _RopeQK.apply(_own_storage(q), _own_storage(k), cu_seqlens, float(theta), seqused,
                         position_ids, seq_offsets, float(pos_scale), bool(inplace_backward),
                         cu_valid, valid)


def _qkv_split(qkv: torch.Tensor, Hq: int, Hkv: int):
    """Q and K views [T, Hq, D] and [T, Hkv, D] of a fused projection output
    [T, (Hq + 2 Hkv) * D] or [T, Hq + 2 Hkv, D] whose columns are contiguous."""
    H = Hq + 2 * Hkv
    if qkv.dim() == 3:
        if qkv.shape[1] != H:
            raise ValueError(f"qkv has {qkv.shape[1]} heads, expected Hq + 2 Hkv = {H}")
        if (qkv.shape[2] > 1 and qkv.stride(2) != 1) or (H > 1 and qkv.stride(1) != qkv.shape[2]):
            raise ValueError("qkv: the heads of a token must be contiguous")
        flat = qkv.flatten(1)
    elif qkv.dim() == 2:
        if qkv.shape[1] % H:
            raise ValueError(f"qkv has {qkv.shape[1]} columns, not a multiple of Hq + 2 Hkv = {H}")
        if qkv.shape[1] > 1 and qkv.stride(1) != 1:
            raise ValueError("qkv: columns must be contiguous")
        flat = qkv
    else:
        raise ValueError("qkv must be [T, (Hq + 2 Hkv) * D] or [T, Hq + 2 Hkv, D]")
    D = flat.shape[1] // H
    q = flat[:, :Hq * D].unflatten(1, (Hq, D))
    k = flat[:, Hq * D:(Hq + Hkv) * D].unflatten(1, (Hkv, D))
    return q, k


class _RopeQKV(torch.autograd.Function):
    @staticmethod
    def forward(ctx, qkv, Hq, Hkv, cu_seqlens, theta, seqused, position_ids, seq_offsets,
                pos_scale, inplace_backward, cu_valid, valid_tokens):
        q, k = _qkv_split(qkv, Hq, Hkv)
        _rotate(q, k, theta, 1, cu_seqlens, seqused, position_ids, seq_offsets, pos_scale,
                cu_valid, valid_tokens)
        ctx.mark_dirty(qkv)
        ctx.save_for_backward(cu_seqlens, seqused, position_ids, seq_offsets, cu_valid)
        ctx.heads, ctx.theta, ctx.pos_scale = (Hq, Hkv), theta, pos_scale
        ctx.inplace, ctx.valid = inplace_backward, valid_tokens
        return qkv

    @staticmethod
    def backward(ctx, g):
        cu, su, pid, so, cv = ctx.saved_tensors
        if not (ctx.inplace and g.is_contiguous()):
            g = g.clone(memory_format=torch.contiguous_format)
        dq, dk = _qkv_split(g, *ctx.heads)
        _rotate(dq, dk, ctx.theta, -1, cu, su, pid, so, ctx.pos_scale, cv, ctx.valid)
        return g, None, None, None, None, None, None, None, None, None, None, None


def rope_qkv(qkv: torch.Tensor, num_q_heads: int, num_kv_heads: int, cu_seqlens=None,
             theta: float = 10000.0, seqused=None, position_ids=None, seq_offsets=None,
             pos_scale: float = 1.0, inplace_backward: bool = False, cu_valid=None,
             valid_tokens=None) -> torch.Tensor:
    """Differentiable in-place RoPE of the Q and K heads inside a fused QKV projection
    output qkv [T, (Hq + 2 Hkv) * D] or [T, Hq + 2 Hkv, D] (Q heads, then K, then V;
    each token's columns contiguous, rows of any stride), one kernel launch per
    pass; the V heads and their gradient pass through unchanged. qkv may be a view
    (e.g. ``(x @ W_qkv).view(T, -1, D)``). Positions (and the compact padded launch)
    as in ``rope_qk``. Returns qkv."""
    valid = _padded_args(position_ids, cu_valid, valid_tokens)
    return _RopeQKV.apply(qkv, int(num_q_heads), int(num_kv_heads), cu_seqlens, float(theta),
                          seqused, position_ids, seq_offsets, float(pos_scale),
                          bool(inplace_backward), cu_valid, valid)


class _RopeQKTable(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, cos_tab, sin_tab, cu_seqlens, seqused, position_ids, seq_offsets,
                inplace_backward):
        qk_apply_table_(q, k, cos_tab, sin_tab, 1, cu_seqlens=cu_seqlens, seqused=seqused,
                        seq_offsets=seq_offsets, position_ids=position_ids)
        ctx.mark_dirty(q, k)
        ctx.save_for_backward(cos_tab, sin_tab, cu_seqlens, seqused, position_ids, seq_offsets)
        ctx.inplace = inplace_backward
        return q, k

    @staticmethod
    def backward(ctx, dq, dk):
        ct, st, cu, su, pid, so = ctx.saved_tensors
        if not (ctx.inplace and dq.is_contiguous()):
            dq = dq.clone(memory_format=torch.contiguous_format)
        if not (ctx.inplace and dk.is_contiguous()):
            dk = dk.clone(memory_format=torch.contiguous_format)
        qk_apply_table_(dq, dk, ct, st, -1, cu_seqlens=cu, seqused=su, seq_offsets=so,
                        position_ids=pid)
        return dq, dk, None, None, None, None, None, None, None


def rope_qk_table(q: torch.Tensor, k: torch.Tensor, cos_tab: torch.Tensor, sin_tab: torch.Tensor,
                  cu_seqlens=None, seqused=None, position_ids=None, seq_offsets=None,
                  inplace_backward: bool = False):
    """rope_qk with cos/sin read from float32 [rows, D/2] tables (row p = position p,
    as ``qk_apply_table_`` takes them) instead of computed from theta (views that
    require grad are rotated on copies, as in rope_qk). The tables are
    constants: they receive no gradient. Tokens whose position has no row pass
    through unchanged, and so do their gradients."""
    return _RopeQKTable.apply(_own_storage(q), _own_storage(k), cos_tab, sin_tab, cu_seqlens,
                              seqused, position_ids, seq_offsets, bool(inplace_backward))


class _Glu(torch.autograd.Function):
    @staticmethod
    def forward(ctx, kind, e, g):
        ctx.kind = kind
        ctx.save_for_backward(e, g)
        return glu_fwd(kind, e, g)

    @staticmethod
    def backward(ctx, dh):
        e, g = ctx.saved_tensors
        de, dg = glu_bwd(ctx.kind, dh.contiguous(), e, g)
        return None, de, dg


def glu(kind: str, e: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """Differentiable h = act(e) * g, act = silu ("swiglu"), exact gelu ("geglu")
    or tanh gelu ("geglu_tanh"); e, g [rows, cols] with contiguous columns and one
    row stride."""
    return _Glu.apply(kind, e, g)


class _GluFused(torch.autograd.Function):
    @staticmethod
    def forward(ctx, kind, gate_up):
        cols = gate_up.shape[1] // 2
        ctx.kind, ctx.cols = kind, cols
        ctx.save_for_backward(gate_up)
        return glu_fwd(kind, gate_up[:, :cols], gate_up[:, cols:])

    @staticmethod
    def backward(ctx, dh):
        (gate_up,) = ctx.saved_tensors
        cols = ctx.cols
        grad = torch.empty_like(gate_up, memory_format=torch.contiguous_format)
        glu_bwd(ctx.kind, dh.contiguous(), gate_up[:, :cols], gate_up[:, cols:],
                de=grad[:, :cols], dg=grad[:, cols:])
        return None, grad


def glu_fused(kind: str, gate_up: torch.Tensor) -> torch.Tensor:
    """glu() on the two halves of one fused gate/up projection output
    gate_up [rows, 2 * cols] (gate first); the gradient is one [rows, 2 * cols]
    tensor written by a single backward launch."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [rows, 2 * cols]")
    if not gate_up.is_contiguous():
        raise ValueError("gate_up must be contiguous")
    return _GluFused.apply(kind, gate_up)
