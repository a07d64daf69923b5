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
)

__all__ = [
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
]
