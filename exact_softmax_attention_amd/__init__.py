"""Exact softmax attention, forward and backward (FlashAttention-2 style), on AMD MI355X (gfx950).

Thin ctypes binding over libfa2.so, whose C ABI is declared in include/fa2.h. This module
only marshals arguments: it checks tensor metadata, allocates outputs with torch, passes
raw device pointers and torch's current HIP stream, and turns status codes into
exceptions. Every step of the computation runs in the HIP kernels; there is no fallback.
"""
from __future__ import annotations

from ._lib import (
    FA2_ABI_VERSION,
    Fa2Error,
    STATUS,
    bwd,
    bwd_varlen,
    fwd,
    fwd_chunk,
    fwd_gqa,
    fwd_splitkv,
    fwd_varlen,
    fwd_varlen_gqa,
    geometry,
    lib_path,
    load_library,
    lse_merge,
    num_variants,
    variant_name,
    varlen_default_variant,
)


def attention(*args, **kwargs):
    """Differentiable attention (autograd reaches the library's backward); see
    ``exact_softmax_attention_amd.autograd.attention``."""
    from .autograd import attention as _attention
    return _attention(*args, **kwargs)


def attention_varlen(*args, **kwargs):
    """Differentiable packed variable-length attention; see
    ``exact_softmax_attention_amd.autograd.attention_varlen``."""
    from .autograd import attention_varlen as _attention_varlen
    return _attention_varlen(*args, **kwargs)

__all__ = [
    "attention",
    "attention_varlen",
    "FA2_ABI_VERSION",
    "Fa2Error",
    "STATUS",
    "bwd",
    "bwd_varlen",
    "fwd",
    "fwd_chunk",
    "fwd_gqa",
    "fwd_splitkv",
    "fwd_varlen",
    "fwd_varlen_gqa",
    "geometry",
    "lib_path",
    "load_library",
    "lse_merge",
    "num_variants",
    "variant_name",
    "varlen_default_variant",
]
