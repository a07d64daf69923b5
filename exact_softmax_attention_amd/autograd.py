"""torch.autograd functions over the library's forward and backward entry points.

``attention(q, k, v)`` returns O = softmax(scale·QKᵀ [causal mask])·V and lets torch's
autograd reach dQ, dK and dV through the library's backward (the pages' Algorithm 2: P is
recomputed from the stored LSE, with D = rowsum(dO∘O)). Both directions run in the HIP
kernels. This module saves Q, K, V, O and the LSE for the backward, and otherwise only
forwards arguments: no arithmetic of the method happens here. Grouped-query K/V (H_kv
dividing H) and packed variable-length batches (``attention_varlen``) are supported as in
the forward.
"""
from __future__ import annotations

import torch

from . import _lib


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = _lib.fwd_gqa(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, causal, scale):
        o, lse = _lib.fwd_varlen_gqa(q, k, v, cu_seqlens, max_seqlen, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.max_seqlen, ctx.causal, ctx.scale = max_seqlen, causal, scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse, cu = ctx.saved_tensors
        dq, dk, dv = _lib.bwd_varlen(q, k, v, o, lse, do.contiguous(), cu, ctx.max_seqlen,
                                     causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, causal: bool = False, scale: float | None = None, return_lse: bool = False):
    """Differentiable attention over bf16 GPU tensors q [B, H, N, d], k/v [B, H_kv, N, d].

    Returns O [B, H, N, d] (and the LSE [B, H, N], which carries no gradient, when
    ``return_lse``). ``scale`` defaults to 1/sqrt(d)."""
    o, lse = _Attention.apply(q, k, v, bool(causal), scale)
    return (o, lse) if return_lse else o


def attention_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
                     return_lse: bool = False):
    """Differentiable attention over a packed variable-length batch: q [H, T, d], k/v
    [H_kv, T, d] bf16, ``cu_seqlens`` int32 [num_seqs + 1] on the GPU."""
    o, lse = _AttentionVarlen.apply(q, k, v, cu_seqlens, int(max_seqlen), bool(causal), scale)
    return (o, lse) if return_lse else o
