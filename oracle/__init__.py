"""CPU fp64 oracle for exact softmax attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. The product path never does.
"""
from .attention import (attention, attention_chunk, attention_chunk_head, lse_merge, attention_backward_gqa, attention_backward_head, attention_backward_varlen,
                        attention_gqa, attention_head, attention_rows, attention_varlen, attention_varlen_gqa,
                        kv_head)

__all__ = ["attention", "attention_chunk", "attention_chunk_head", "lse_merge", "attention_backward_gqa", "attention_backward_head", "attention_backward_varlen",
           "attention_gqa", "attention_head", "attention_rows", "attention_varlen", "attention_varlen_gqa",
           "kv_head"]
