"""Seeded synthetic inputs for exact softmax attention.

This module is shared by both sides of every comparison (the CPU fp64 oracle
and the gfx950 kernels). It only draws random numbers and describes the
workloads; it contains none of the attention arithmetic.

Workloads follow the micro-benchmark of the FlashAttention-2 paper summary
(paper-graph-ui page, "5. Experimental Analysis", "Evaluation Methodology"):
synthetic Q, K, V, 16k total tokens, hidden size 2048, head dimension 64 or
128, with and without a causal mask. Values are i.i.d. standard normal in
float32, rounded to bfloat16 (round-to-nearest-even) once. Seeds are fixed
per workload so that every run sees the same tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_qkv",
    "make_varlen",
    "varlen_lengths",
    "metric_flops",
]


@dataclass(frozen=True)
class Workload:
    """One benchmark/parity configuration.

    Fixed-length workloads use tensors of shape [B, H, N, d]. The packed
    variable-length workload (``varlen=True``) uses [H, T, d] with
    ``T = sum(lengths)`` and int32 ``cu_seqlens`` offsets of length
    ``num_seqs + 1``.
    """

    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    k_scale: float = 1.0
    varlen: bool = False
    num_seqs: int = 0
    min_len: int = 0
    max_len: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the float32 value the kernel receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())


WORKLOADS: dict[str, Workload] = {
    "single_head_256": Workload("single_head_256", B=1, H=1, N=256, d=64, causal=False, seed=1,
                   description="single head: B=1 H=1 N=256 d=64, non-causal"),
    "batch8_2k_d128": Workload("batch8_2k_d128", B=8, H=16, N=2048, d=128, causal=False, seed=2,
                   description="B=8 H=16 N=2048 d=128 (16k tokens, hidden 2048), non-causal"),
    "batch8_2k_d64_causal": Workload("batch8_2k_d64_causal", B=8, H=32, N=2048, d=64, causal=True, seed=3,
                   description="B=8 H=32 N=2048 d=64 (hidden 2048), causal"),
    "long_16k_causal": Workload("long_16k_causal", B=1, H=16, N=16384, d=128, causal=True, seed=4,
                   description="long context: B=1 H=16 N=16384 d=128, causal"),
    "varlen16_causal": Workload("varlen16_causal", B=1, H=16, N=0, d=128, causal=True, seed=5, k_scale=3.0,
                   varlen=True, num_seqs=16, min_len=128, max_len=4096,
                   description="packed varlen: 16 sequences, lengths U[128,4096], "
                               "H=16 d=128, causal per sequence, K scaled by 3"),
}


def _randn_bf16(shape, gen: torch.Generator, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult  # scaled in float32, then rounded to bf16 once
    return x.to(torch.bfloat16)


def make_qkv(B: int, H: int, N: int, d: int, seed: int, k_scale: float = 1.0, H_kv: int | None = None):
    """Return CPU bf16 tensors q [B, H, N, d] and k, v [B, H_kv, N, d] (drawn in that
    order; H_kv defaults to H)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    H_kv = H if H_kv is None else int(H_kv)
    q = _randn_bf16((B, H, N, d), gen)
    k = _randn_bf16((B, H_kv, N, d), gen, k_scale)
    v = _randn_bf16((B, H_kv, N, d), gen)
    return q, k, v


def varlen_lengths(num_seqs: int, min_len: int, max_len: int, gen: torch.Generator) -> list[int]:
    """Integer lengths drawn uniformly from [min_len, max_len] inclusive."""
    return [int(x) for x in torch.randint(min_len, max_len + 1, (num_seqs,), generator=gen)]


def make_varlen(H: int, d: int, seed: int, lengths=None, num_seqs: int = 16,
                min_len: int = 128, max_len: int = 4096, k_scale: float = 1.0, H_kv: int | None = None):
    """Packed variable-length batch.

    Returns (q, k, v, cu_seqlens, lengths): q is CPU bf16 [H, T, d], k and v
    [H_kv, T, d] (H_kv defaults to H),
    cu_seqlens is an int32 CPU tensor [num_seqs + 1] with cu[0] = 0 and
    cu[s+1] - cu[s] = lengths[s]. If ``lengths`` is None it is drawn first from
    the same generator, then q, k, v are drawn in that order.
    """
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    if lengths is None:
        lengths = varlen_lengths(num_seqs, min_len, max_len, gen)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    H_kv = H if H_kv is None else int(H_kv)
    q = _randn_bf16((H, T, d), gen)
    k = _randn_bf16((H_kv, T, d), gen, k_scale)
    v = _randn_bf16((H_kv, T, d), gen)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, cu, lengths


def workload_inputs(w: Workload):
    """Inputs for a named workload: (q, k, v) or (q, k, v, cu_seqlens, lengths)."""
    if w.varlen:
        return make_varlen(w.H, w.d, w.seed, num_seqs=w.num_seqs, min_len=w.min_len,
                           max_len=w.max_len, k_scale=w.k_scale)
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.k_scale)


def metric_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """The benchmark's FLOP count: 4*B*H*N^2*d, halved for causal.

    This is the paper's accounting for forward attention (paper-graph-ui page,
    "Evaluation Methodology", Metrics bullet; chlience notes, "Result 1"):
    two matmuls of 2*N^2*d each per head, causal counted as exactly one half.
    """
    f = 4.0 * B * H * float(N) * float(N) * d
    return f / 2.0 if causal else f


def varlen_metric_flops(lengths, H: int, d: int, causal: bool) -> float:
    """Sum over packed sequences of the per-sequence metric FLOPs."""
    return sum(metric_flops(1, H, int(n), d, causal) for n in lengths)
