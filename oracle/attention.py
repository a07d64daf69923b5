"""CPU fp64 oracle for exact softmax attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
kernels and imports nothing from the product package.

What it computes. The pages state that FlashAttention-2 is exact: it changes
how attention is executed, not what it computes (chlience notes, "阅读目标与判断
边界" and §5; paper-graph-ui summary, §3.4 "Algorithm 1 Walkthrough",
"Mathematical correctness"). So this oracle is the plain, materialised
definition, written out once per head with no tiling:

    S = scale * Q K^T                          (N x N)
    S[i, j] = -inf  where causal and j > i
    m_i = max_j S[i, j]
    l_i = sum_j exp(S[i, j] - m_i)
    P = exp(S - m) / l                         (row softmax)
    O = P V
    LSE_i = m_i + ln(l_i)

Sources for each line:
  * S = Q K^T, P = softmax(S), O = P V: chlience notes §1 (研究问题、背景和价值);
    the 1/sqrt(d) scale inside the score: llm-infra-atlas "FlashAttention" §1
    (为什么 attention 是 memory-bound). The scale is a parameter here.
  * the two-pass safe softmax (row max, sum of exp(S - m), divide):
    paper-graph-ui summary §3.4, "FlashAttention's Online Softmax", the
    standard (non-online) three-step approach.
  * LSE = m + log(l), natural log: chlience notes §5.2 (算法语义层);
    paper-graph-ui §3.4, "Tweak 2: Store Logsumexp".
  * causal: entries with column index greater than row index are -inf:
    paper-graph-ui §3.4, "Causal masking optimization"; chlience notes §5.6.
  * grouped/multi-query attention: query head h uses key/value head
    floor(h / g), g = H_q / H_kv query heads per key/value head, K and V never
    copied: chlience notes §5.6 (the MQA/GQA head index mapping).

Readings where the pages are silent:
  * the scale multiplies Q K^T before the softmax, and LSE is taken over the
    scaled scores, in natural log;
  * the scale is the float32 value the kernel receives, widened to fp64;
  * a row with no allowed key (cannot happen for square causal or
    non-causal attention) would give O = 0 and LSE = -inf.

The backward (gradients with respect to Q, K, V) is the same materialised
definition differentiated by hand: chlience notes §5.3, paper-graph-ui §3.4
"The Backward Pass: Simpler Statistics, Same Structure".

Every function here is pinned by tests/test_oracle_pins.py (brute force,
closed forms, library routines, invariants and the pages' online
recurrence); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention", "attention_chunk", "attention_chunk_head", "lse_merge", "attention_backward_gqa", "attention_backward_head", "attention_backward_varlen",
           "attention_gqa", "attention_head", "attention_rows", "attention_varlen", "attention_varlen_gqa",
           "kv_head"]


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(s: np.ndarray):
    """Two-pass safe softmax of each row of s (entries may be -inf).

    Returns (P, LSE). Rows whose entries are all -inf give P = 0, LSE = -inf.
    """
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)                # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l > 0.0, e / np.where(l > 0.0, l, 1.0), 0.0)
        lse = np.where(l[:, 0] > 0.0, m_safe[:, 0] + np.log(np.where(l[:, 0] > 0.0, l[:, 0], 1.0)),
                       -np.inf)
    return p, lse


def attention_head(q, k, v, causal: bool, scale: float):
    """Exact attention for one head.

    q, k, v: [N, d] arrays (converted to float64). Returns (O [N, d],
    LSE [N]) in float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    n = q.shape[0]
    if n == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    s = float(scale) * (q @ k.T)
    if causal:
        s[np.triu_indices(n, k=1)] = -np.inf     # key index j > query index i
    p, lse = _softmax_rows(s)
    return p @ v, lse


def attention(q, k, v, causal: bool, scale: float):
    """Exact attention over [B, H, N, d] inputs; returns (O [B,H,N,d], LSE [B,H,N])."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, _ = q.shape
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, rows):
    """Exact attention for selected query rows of one head.

    The softmax is per row, so row i of the result needs only q_i and all of
    K and V; this evaluates the same definition as ``attention_head`` on a
    subset of rows (used to check very large problems one row at a time).
    q, k, v: [N, d]. rows: integer indices into [0, N). Returns
    (O [len(rows), d], LSE [len(rows)]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    n = k.shape[0]
    s = float(scale) * (q[rows] @ k.T)
    if causal:
        s[np.arange(n)[None, :] > rows[:, None]] = -np.inf
    p, lse = _softmax_rows(s)
    return p @ v, lse


def attention_varlen(q, k, v, cu_seqlens, causal: bool, scale: float):
    """Exact attention over a packed batch of sequences.

    q, k, v: [H, T, d]; cu_seqlens: [S + 1] offsets with cu[0] = 0 and
    cu[S] = T. Sequence s occupies tokens [cu[s], cu[s+1]) of every head and
    attends only within itself; the causal mask uses indices local to the
    sequence. Returns (O [H, T, d], LSE [H, T]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    H, T, _ = q.shape
    o = np.zeros(q.shape[:2] + (v.shape[2],))
    lse = np.zeros((H, T))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            o[h, a:b], lse[h, a:b] = attention_head(q[h, a:b], k[h, a:b], v[h, a:b], causal, scale)
    return o, lse


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h: floor(h / g) with g = H / H_kv (chlience §5.6)."""
    if H_kv <= 0 or H % H_kv:
        raise ValueError(f"H_kv={H_kv} must divide H={H}")
    return h // (H // H_kv)


def attention_gqa(q, k, v, causal: bool, scale: float):
    """Grouped-query attention: q [B, H, N, d]; k, v [B, H_kv, N, d] with H_kv | H.

    Each query head is the plain definition (``attention_head``) against the
    key/value head ``kv_head`` maps it to. Returns (O [B,H,N,d], LSE [B,H,N]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, _ = q.shape
    H_kv = k.shape[1]
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, hk], v[b, hk], causal, scale)
    return o, lse


def attention_varlen_gqa(q, k, v, cu_seqlens, causal: bool, scale: float):
    """Packed grouped-query attention: q [H, T, d]; k, v [H_kv, T, d]; sequences as in
    ``attention_varlen``. Returns (O [H, T, d], LSE [H, T])."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    H, T, _ = q.shape
    H_kv = k.shape[0]
    o = np.zeros(q.shape[:2] + (v.shape[2],))
    lse = np.zeros((H, T))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            o[h, a:b], lse[h, a:b] = attention_head(q[h, a:b], k[hk, a:b], v[hk, a:b], causal, scale)
    return o, lse


# ---------------------------------------------------------------------------
# Backward (gradients of O with respect to Q, K, V for an upstream gradient dO)
# ---------------------------------------------------------------------------

def attention_backward_head(q, k, v, do, causal: bool, scale: float):
    """Gradients of O = softmax(scale * Q K^T [causal]) V for one head, from the definition.

    With P the materialised softmax (``_softmax_rows``) and O = P V:
        dV = P^T dO,   dP = dO V^T,   D = rowsum(dO o O),   dS = P o (dP - D),
        dQ = scale * dS K,   dK = scale * dS^T Q
    (chlience notes §5.3; paper-graph-ui §3.4 "The Backward Pass: Simpler Statistics, Same
    Structure", which also derives D = rowsum(P o dP) = rowsum(dO o O) from the softmax
    Jacobian). The pages write dQ = dS K, dK = dS^T Q for an unscaled score; the factor
    ``scale`` is the chain rule through S = scale * Q K^T. Masked entries have P = 0 and so
    dS = 0. q, k, v, do: [N, d]; returns (dQ, dK, dV) in float64.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    n = q.shape[0]
    if n == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    s = float(scale) * (q @ k.T)
    if causal:
        s[np.triu_indices(n, k=1)] = -np.inf
    p, _ = _softmax_rows(s)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    dvec = np.sum(do * o, axis=1, keepdims=True)
    ds = p * (dp - dvec)
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward_gqa(q, k, v, do, causal: bool, scale: float):
    """Backward over q, do [B, H, N, d] and k, v [B, H_kv, N, d] (H_kv | H): the gradient of a
    key/value head is the sum over the query heads mapped to it (chlience notes §5.6).
    Returns (dQ [B,H,N,d], dK [B,H_kv,N,d], dV [B,H_kv,N,d])."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            gq, gk, gv = attention_backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], causal, scale)
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_seqlens, causal: bool, scale: float):
    """Packed backward: q, do [H, T, d]; k, v [H_kv, T, d]; sequences as in
    ``attention_varlen``. Returns (dQ, dK, dV)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    H = q.shape[0]
    H_kv = k.shape[0]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            gq, gk, gv = attention_backward_head(q[h, a:b], k[hk, a:b], v[hk, a:b], do[h, a:b], causal, scale)
            dq[h, a:b] = gq
            dk[hk, a:b] += gk
            dv[hk, a:b] += gv
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Key/value chunks and the merge of partial results by their logsumexp
# ---------------------------------------------------------------------------

def attention_chunk_head(q, k, v, causal: bool, diag: int, scale: float):
    """Attention of q [N_q, d] over one key/value chunk k, v [N_k, d].

    Causal: query i may attend key j iff j <= i + diag (for the chunk [a, b) of a sequence
    whose queries start at position q0, diag = q0 - a). Rows with no allowed key give O = 0
    and LSE = -inf. The plain definition, as ``attention_head``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    nq, nk = q.shape[0], k.shape[0]
    if nq == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    if nk == 0:
        return np.zeros((nq, v.shape[1])), np.full((nq,), -np.inf)
    s = float(scale) * (q @ k.T)
    if causal:
        s[np.arange(nk)[None, :] > np.arange(nq)[:, None] + int(diag)] = -np.inf
    p, lse = _softmax_rows(s)
    return p @ v, lse


def attention_chunk(q, k, v, causal: bool, diag: int, scale: float):
    """``attention_chunk_head`` over q [B, H, N_q, d] and k, v [B, H_kv, N_k, d]."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, nq, _ = q.shape
    H_kv = k.shape[1]
    o = np.zeros((B, H, nq, v.shape[3]))
    lse = np.zeros((B, H, nq))
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = attention_chunk_head(q[b, h], k[b, hk], v[b, hk], causal, diag, scale)
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge partial results over disjoint key sets (llm-infra-atlas "FlashAttention" §5 and
    the LSE mix of its §0 reading table): LSE = log sum_s exp(LSE_s),
    O = sum_s exp(LSE_s - LSE) O_s. o_parts [S, ..., d], lse_parts [S, ...]; rows whose LSE_s
    are all -inf give O = 0, LSE = -inf. Returns (O [..., d], LSE [...]) in float64."""
    o_parts, lse_parts = _as_f64(o_parts), _as_f64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])               # exp(-inf) = 0
    z = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
        wn = np.where(z[None] > 0, w / np.where(z > 0, z, 1.0)[None], 0.0)
    o = np.sum(wn[..., None] * o_parts, axis=0)
    return o, lse
