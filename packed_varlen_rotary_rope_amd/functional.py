"""Autograd entry points over the C ABI: the packed-varlen QK rotary embedding
and the SwiGLU / GeGLU activations as differentiable torch functions.

Every pass is one launch of the library's kernels on the current stream; this
module only wires them into torch.autograd (no arithmetic of its own).

    q, k = rope_qk(q, k, cu_seqlens, theta)        # in place, returns q and k
    q, k = rope_qk_table(q, k, cos_tab, sin_tab, cu_seqlens)  # cos/sin from tables
    h = glu("swiglu", e, g)                        # h = silu(e) * g
    h = glu_fused("geglu", gate_up)                # e, g = halves of gate_up

rope_qk rotates its inputs in place (they are marked dirty), so q and k must not
be leaf tensors that require grad -- in a model they are projection outputs. Its
backward applies the transposed rotation (sin negated, Unsloth, "Entrainement des
LLM 3 fois plus rapide...", fused QK RoPE section) to the incoming gradients:
in place on them when ``inplace_backward=True``, otherwise on a copy, because
autograd may hand the same gradient tensor to several consumers (an addition
passes its gradient to both operands), and rotating a shared tensor in place
would change the other consumer's gradient.
"""
from __future__ import annotations

import torch

from . import glu_bwd, glu_fwd, qk_apply_ex_, qk_apply_table_


class _RopeQK(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, cu_seqlens, theta, seqused, position_ids, seq_offsets, pos_scale,
                inplace_backward):
        qk_apply_ex_(q, k, theta, 1, cu_seqlens=cu_seqlens, seqused=seqused,
                     seq_offsets=seq_offsets, position_ids=position_ids, pos_scale=pos_scale)
        ctx.mark_dirty(q, k)
        ctx.save_for_backward(cu_seqlens, seqused, position_ids, seq_offsets)
        ctx.theta, ctx.pos_scale, ctx.inplace = theta, pos_scale, inplace_backward
        return q, k

    @staticmethod
    def backward(ctx, dq, dk):
        # gradients that did not flow arrive as zeros (materialized by autograd)
        cu, su, pid, so = ctx.saved_tensors
        if not (ctx.inplace and dq.is_contiguous()):
            dq = dq.clone(memory_format=torch.contiguous_format)
        if not (ctx.inplace and dk.is_contiguous()):
            dk = dk.clone(memory_format=torch.contiguous_format)
        qk_apply_ex_(dq, dk, ctx.theta, -1, cu_seqlens=cu, seqused=su, seq_offsets=so,
                     position_ids=pid, pos_scale=ctx.pos_scale)
        return dq, dk, None, None, None, None, None, None, None


def rope_qk(q: torch.Tensor, k: torch.Tensor, cu_seqlens=None, theta: float = 10000.0,
            seqused=None, position_ids=None, seq_offsets=None, pos_scale: float = 1.0,
            inplace_backward: bool = False):
    """Differentiable in-place RoPE of q [T, Hq, D] and k [T, Hkv, D] (views with
    contiguous heads, e.g. slices of a fused QKV output, are accepted). Positions
    come from cu_seqlens (with optional seqused / seq_offsets) or position_ids, as
    in ``qk_apply_ex_``. Returns (q, k), rotated."""
    return _RopeQK.apply(q, k, cu_seqlens, float(theta), seqused, position_ids, seq_offsets,
                         float(pos_scale), bool(inplace_backward))


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
    as ``qk_apply_table_`` takes them) instead of computed from theta. The tables are
    constants: they receive no gradient. Tokens whose position has no row pass
    through unchanged, and so do their gradients."""
    return _RopeQKTable.apply(q, k, cos_tab, sin_tab, cu_seqlens, seqused, position_ids,
                              seq_offsets, bool(inplace_backward))


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
