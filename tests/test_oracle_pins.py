"""Pins for the CPU fp64 oracle (no GPU needed).

The pages print no numeric outputs for any input, so the oracle is pinned to
things other than itself:

  * brute force on tiny inputs with scalar Python loops (math.exp, math.fsum),
    without the max-subtraction trick;
  * an independent library implementation (torch's float64 CPU
    scaled_dot_product_attention; scipy's logsumexp);
  * closed forms: identical V rows, Q = 0, causal row 0, length-1 sequences,
    one-hot attention through orthogonal keys, extreme scores;
  * invariants the pages fix: P = exp(S - LSE) sums to 1 per row (chlience
    notes §5.2; paper-graph-ui §3.4 "Tweak 2"), max S <= LSE <= max S + ln n,
    O inside the hull of the allowed V rows, joint key/value permutation,
    row-constant score shifts;
  * the pages' own one-pass recurrence — FA2's unscaled accumulator with a
    single final division (chlience notes §5.2; paper-graph-ui §3.4
    "Algorithm 1 Walkthrough") and FA1's renormalising form (paper-graph-ui
    §3.4 "FlashAttention's Online Softmax") — equals the two-pass oracle for
    block sizes 1, 3 and 64, with and without causal block skipping;
  * a mutation check: copies of the oracle with one planted mistake each
    (dropped scale, dropped max in the LSE, wrong mask edge or triangle,
    softmax over the wrong axis, transposed operands, no max subtraction)
    must each fail at least one of these pins.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import (attention, attention_gqa, attention_head, attention_rows, attention_varlen,
                    attention_varlen_gqa, kv_head)

RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Pin implementations, parametrised by the per-head implementation under test
# so that the mutation check can run them against planted mistakes.
# Each returns None on success or a string describing the failure.
# ---------------------------------------------------------------------------

def _brute_force(q, k, v, causal, scale):
    """Scalar Python loops: w_j = exp(S_ij) directly (no max subtraction)."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        js = [j for j in range(n) if (not causal or j <= i)]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in js}
        w = {j: math.exp(s[j]) for j in js}
        z = math.fsum(w.values())
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in js) / z
        lse[i] = math.log(z)
    return np.array(o), np.array(lse)


def pin_brute_force(impl):
    rng = np.random.default_rng(7)
    for n in (1, 2, 3, 5, 8):
        for d in (1, 2, 4):
            for causal in (False, True):
                for mag in (1.0, 6.0):   # mag 6 with d=4 gives scores up to ~+-60
                    q = rng.standard_normal((n, d)) * mag
                    k = rng.standard_normal((n, d)) * mag
                    v = rng.standard_normal((n, 3))
                    scale = 0.7
                    o_ref, l_ref = _brute_force(q.tolist(), k.tolist(), v.tolist(), causal, scale)
                    o, l = impl(q, k, v, causal, scale)
                    if not (np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)
                            and np.allclose(l, l_ref, rtol=1e-13, atol=1e-12)):
                        return f"brute force mismatch n={n} d={d} causal={causal} mag={mag}"
    return None


def pin_library_sdpa(impl):
    """torch float64 CPU scaled_dot_product_attention (math path) as a second implementation."""
    rng = np.random.default_rng(8)
    for n, d, causal in ((37, 16, False), (37, 16, True), (64, 8, True), (5, 64, False)):
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        scale = 1.0 / math.sqrt(d) * 1.3
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
            torch.from_numpy(v)[None, None], is_causal=causal, scale=scale)[0, 0].numpy()
        scores = np.einsum("id,jd->ij", q, k) * scale
        if causal:
            scores = np.where(np.tril(np.ones((n, n), dtype=bool)), scores, -np.inf)
        lse_ref = scipy.special.logsumexp(scores, axis=1)
        o, l = impl(q, k, v, causal, scale)
        if not (np.allclose(o, ref, rtol=1e-11, atol=1e-12) and np.allclose(l, lse_ref, rtol=1e-12, atol=1e-12)):
            return f"library mismatch n={n} d={d} causal={causal}"
    return None


def pin_identical_v_rows(impl):
    rng = np.random.default_rng(9)
    for causal in (False, True):
        n, d = 33, 8
        q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        row = rng.standard_normal(5)
        v = np.tile(row, (n, 1))
        o, _ = impl(q, k, v, causal, 0.4)
        if not np.allclose(o, np.tile(row, (n, 1)), rtol=0, atol=1e-13):
            return f"identical V rows not reproduced (causal={causal})"
    return None


def pin_zero_q(impl):
    rng = np.random.default_rng(10)
    n, d = 19, 6
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, 4))
    q = np.zeros((n, d))
    o, l = impl(q, k, v, False, 0.9)
    if not (np.allclose(o, np.tile(v.mean(axis=0), (n, 1)), atol=1e-13)
            and np.allclose(l, np.full(n, math.log(n)), atol=1e-13)):
        return "Q=0 non-causal: O != mean(V) or LSE != ln N"
    o, l = impl(q, k, v, True, 0.9)
    cummean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    if not (np.allclose(o, cummean, atol=1e-13)
            and np.allclose(l, np.log(np.arange(1, n + 1)), atol=1e-13)):
        return "Q=0 causal: O != prefix mean(V) or LSE != ln(i+1)"
    return None


def pin_causal_row0(impl):
    rng = np.random.default_rng(11)
    n, d = 24, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 0.35
    o, l = impl(q, k, v, True, scale)
    if not (np.allclose(o[0], v[0], atol=1e-14) and abs(l[0] - scale * float(np.dot(q[0], k[0]))) < 1e-13):
        return "causal row 0: O_0 != V_0 or LSE_0 != scale*q0.k0"
    # the last causal row sees every key, like the non-causal row
    o2, l2 = impl(q, k, v, False, scale)
    if not (np.allclose(o[-1], o2[-1], atol=1e-13) and abs(l[-1] - l2[-1]) < 1e-12):
        return "causal last row differs from non-causal last row"
    return None


def pin_one_hot(impl):
    """Orthonormal keys and q_i = a * k_{pi(i)}: the softmax is one-hot at pi(i).

    With a permutation pi that is not an involution, this separates Q from K
    and S from its transpose.
    """
    n = 6
    k = np.eye(n)
    perm = np.array([2, 0, 5, 1, 3, 4])
    q = 200.0 * k[perm]
    v = np.random.default_rng(12).standard_normal((n, 3))
    o, l = impl(q, k, v, False, 1.0)
    if not (np.allclose(o, v[perm], atol=1e-12) and np.allclose(l, 200.0, atol=1e-12)):
        return "one-hot attention through orthogonal keys wrong"
    return None


def pin_extreme_scores(impl):
    """Scores of +-1600: the result is the mean of V over the arg-max keys.

    exp(1600) overflows fp64, so this fails unless the row max is subtracted.
    """
    n = 8
    q = np.zeros((n, 2)); q[:, 0] = 40.0
    k = np.zeros((n, 2)); k[:, 0] = np.where(np.arange(n) % 3 == 0, 40.0, -40.0)
    v = np.random.default_rng(13).standard_normal((n, 3))
    o, l = impl(q, k, v, False, 1.0)
    top = np.arange(n) % 3 == 0
    if not (np.all(np.isfinite(o)) and np.allclose(o, np.tile(v[top].mean(axis=0), (n, 1)), atol=1e-12)
            and np.allclose(l, 1600.0 + math.log(top.sum()), atol=1e-10)):
        return "extreme scores not handled"
    return None


def pin_lse_invariants(impl):
    rng = np.random.default_rng(14)
    for causal in (False, True):
        n, d = 40, 16
        q, k = rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)) * 2
        v = rng.standard_normal((n, d))
        scale = 0.25
        o, l = impl(q, k, v, causal, scale)
        s = scale * np.einsum("id,jd->ij", q, k)
        allowed = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
        s = np.where(allowed, s, -np.inf)
        tot = np.exp(s - l[:, None]).sum(axis=1)
        if not np.allclose(tot, 1.0, atol=1e-13):
            return f"sum_j exp(S_ij - LSE_i) != 1 (causal={causal})"
        mx = s.max(axis=1)
        cnt = allowed.sum(axis=1)
        if not (np.all(l >= mx - 1e-12) and np.all(l <= mx + np.log(cnt) + 1e-12)):
            return f"LSE outside [max S, max S + ln n] (causal={causal})"
        for i in range(n):
            vv = v[allowed[i]]
            if not (np.all(o[i] >= vv.min(axis=0) - 1e-12) and np.all(o[i] <= vv.max(axis=0) + 1e-12)):
                return f"O row {i} outside the hull of allowed V rows"
    return None


def pin_permutation(impl):
    rng = np.random.default_rng(15)
    n, d = 29, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o1, l1 = impl(q, k, v, False, 0.5)
    o2, l2 = impl(q, k[perm], v[perm], False, 0.5)
    if not (np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-12)):
        return "not invariant under a joint permutation of key/value rows"
    return None


def pin_row_shift(impl):
    """Adding c to every key adds the row constant scale*q_i.c to S: O unchanged, LSE shifted."""
    rng = np.random.default_rng(16)
    for causal in (False, True):
        n, d = 21, 8
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        c = rng.standard_normal(d) * 3
        o1, l1 = impl(q, k, v, causal, 0.6)
        o2, l2 = impl(q, k + c, v, causal, 0.6)
        if not (np.allclose(o1, o2, atol=1e-12) and np.allclose(l2 - l1, 0.6 * q @ c, atol=1e-12)):
            return f"row-constant shift changed O or LSE wrongly (causal={causal})"
    return None


def pin_scale(impl):
    rng = np.random.default_rng(17)
    n, d = 17, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o1, l1 = impl(q, k, v, True, 0.5)
    o2, l2 = impl(4.0 * q, k, v, True, 0.125)
    o3, _ = impl(q, k, v, True, 0.05)
    if not (np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-12)):
        return "scale does not act on Q K^T"
    if np.allclose(o1, o3, atol=1e-3):
        return "scale has no effect"
    return None


def _fa2_online(q, k, v, causal, scale, br, bc):
    """The pages' one-pass forward, in fp64, for one head.

    Row blocks of br queries are the outer loop; column blocks of bc keys the
    inner loop (chlience notes §5.1 and §5.4; paper-graph-ui §3.4 "Algorithm 1
    Walkthrough"). Per row block the state is the running max m, the running
    sum l and the unscaled accumulator O~; each step takes the new max,
    P~ = exp(S - m_new), rescales l and O~ by exp(m_old - m_new) (a multiply,
    per the languisher erratum for line 10), adds rowsum(P~) and P~ V_j, and
    after the last block divides once by l; LSE = m + log l. With causal,
    column blocks whose first key lies after the block's last query are
    skipped and the mask applies inside the remaining blocks (paper-graph-ui
    §3.4 "Causal masking optimization").
    """
    n, _ = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for r0 in range(0, n, br):
        r1 = min(r0 + br, n)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, v.shape[1]))
        for c0 in range(0, n, bc):
            c1 = min(c0 + bc, n)
            if causal and c0 > r1 - 1:
                break
            s = scale * q[r0:r1] @ k[c0:c1].T
            if causal:
                s = np.where(np.arange(c0, c1)[None, :] > np.arange(r0, r1)[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            p = np.exp(s - m_new[:, None])
            alpha = np.exp(m - m_new)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[c0:c1]
            m = m_new
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def _fa1_online(q, k, v, scale, bc):
    """FA1's form: the output is renormalised after every block (non-causal)."""
    n = q.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, v.shape[1]))
    for c0 in range(0, n, bc):
        s = scale * q @ k[c0:c0 + bc].T
        m_new = np.maximum(m, s.max(axis=1))
        p = np.exp(s - m_new[:, None])
        l_new = np.exp(m - m_new) * l + p.sum(axis=1)
        o = ((l * np.exp(m - m_new))[:, None] * o + p @ v[c0:c0 + bc]) / l_new[:, None]
        m, l = m_new, l_new
    return o, m + np.log(l)


def pin_online_recurrence(impl):
    rng = np.random.default_rng(18)
    n, d = 70, 16
    q, k, v = rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d))
    for causal in (False, True):
        o_ref, l_ref = impl(q, k, v, causal, 0.3)
        for br in (1, 3, 64):
            for bc in (1, 3, 64):
                o, l = _fa2_online(q, k, v, causal, 0.3, br, bc)
                if not (np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)):
                    return f"one-pass FA2 recurrence != oracle (causal={causal}, Br={br}, Bc={bc})"
    o_ref, l_ref = impl(q, k, v, False, 0.3)
    for bc in (1, 3, 64):
        o, l = _fa1_online(q, k, v, 0.3, bc)
        if not (np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)):
            return f"one-pass FA1 recurrence != oracle (Bc={bc})"
    return None


PINS = [pin_brute_force, pin_library_sdpa, pin_identical_v_rows, pin_zero_q, pin_causal_row0,
        pin_one_hot, pin_extreme_scores, pin_lse_invariants, pin_permutation, pin_row_shift,
        pin_scale, pin_online_recurrence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_head_pins(pin):
    assert pin(attention_head) is None


# ---------------------------------------------------------------------------
# Mutation check: each planted mistake must trip at least one pin.
# ---------------------------------------------------------------------------

def _mutant(kind):
    def impl(q, k, v, causal, scale):
        q, k, v = np.asarray(q, float), np.asarray(k, float), np.asarray(v, float)
        n = q.shape[0]
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (k @ q.T if kind == "transpose_s" else q @ k.T)
        if causal:
            tri = {"mask_edge": 0, "mask_triangle": None}.get(kind, 1)
            if kind == "mask_triangle":
                s[np.tril_indices(n, k=-1)] = -np.inf
            else:
                s[np.triu_indices(n, k=tri)] = -np.inf
        axis = 0 if kind == "col_softmax" else 1
        m = s.max(axis=axis, keepdims=True)
        if kind == "no_max":
            m = np.zeros_like(m)
        with np.errstate(all="ignore"):
            e = np.exp(s - m)
            l = e.sum(axis=axis, keepdims=True)
            p = e / l
            o = (p.T @ v) if kind == "transpose_p" else (p @ v)
            lse = np.log(l).ravel() if kind == "lse_no_max" else (m + np.log(l)).ravel()
        return o, lse
    return impl


MUTANTS = ["no_scale", "transpose_s", "mask_edge", "mask_triangle", "col_softmax", "no_max",
           "transpose_p", "lse_no_max"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    impl = _mutant(kind)
    failures = []
    for pin in PINS:
        try:
            r = pin(impl)
        except Exception as e:  # a crash also counts as caught
            r = f"raised {type(e).__name__}"
        if r is not None:
            failures.append(r)
    assert failures, f"no pin caught the planted mistake '{kind}'"


# ---------------------------------------------------------------------------
# The batched, row-subset and packed entry points against the per-head one.
# ---------------------------------------------------------------------------

def test_batched_matches_per_head():
    q, k, v = _rand(2, 3, 20, 8), _rand(2, 3, 20, 8), _rand(2, 3, 20, 8)
    for causal in (False, True):
        o, l = attention(q, k, v, causal, 0.3)
        for b in range(2):
            for h in range(3):
                oh, lh = attention_head(q[b, h], k[b, h], v[b, h], causal, 0.3)
                assert np.array_equal(o[b, h], oh) and np.array_equal(l[b, h], lh)


def test_rows_match_full_head():
    rng = np.random.default_rng(19)
    q, k, v = (rng.standard_normal((50, 8)) for _ in range(3))
    rows = [0, 1, 17, 48, 49]
    for causal in (False, True):
        o, l = attention_head(q, k, v, causal, 0.4)
        orow, lrow = attention_rows(q, k, v, causal, 0.4, rows)
        assert np.allclose(orow, o[rows], atol=1e-14) and np.allclose(lrow, l[rows], atol=1e-14)
        # and against brute force
        ob, lb = _brute_force(q.tolist(), k.tolist(), v.tolist(), causal, 0.4)
        assert np.allclose(orow, ob[rows], atol=1e-12) and np.allclose(lrow, lb[rows], atol=1e-12)


def test_varlen_closed_forms():
    rng = np.random.default_rng(20)
    lengths = [1, 5, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(cu[-1]), 2, 4
    q, k, v = (rng.standard_normal((H, T, d)) for _ in range(3))
    for causal in (False, True):
        o, l = attention_varlen(q, k, v, cu, causal, 0.5)
        for s, n in enumerate(lengths):
            a, b = cu[s], cu[s + 1]
            for h in range(H):
                ob, lb = _brute_force(q[h, a:b].tolist(), k[h, a:b].tolist(), v[h, a:b].tolist(), causal, 0.5)
                assert np.allclose(o[h, a:b], ob, atol=1e-12) and np.allclose(l[h, a:b], lb, atol=1e-12)
            if n == 1:   # a one-token sequence attends only to itself
                assert np.allclose(o[:, a], v[:, a], atol=1e-15)
                assert np.allclose(l[:, a], 0.5 * np.einsum("hd,hd->h", q[:, a], k[:, a]), atol=1e-14)


def test_varlen_single_sequence_equals_fixed():
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((3, 30, 8)) for _ in range(3))
    o1, l1 = attention_varlen(q, k, v, [0, 30], True, 0.3)
    o2, l2 = attention(q[None], k[None], v[None], True, 0.3)
    assert np.array_equal(o1, o2[0]) and np.array_equal(l1, l2[0])


def test_empty_inputs():
    o, l = attention_head(np.zeros((0, 4)), np.zeros((0, 4)), np.zeros((0, 4)), True, 1.0)
    assert o.shape == (0, 4) and l.shape == (0,)
    o, l = attention_varlen(np.zeros((2, 0, 4)), np.zeros((2, 0, 4)), np.zeros((2, 0, 4)), [0], True, 1.0)
    assert o.shape == (2, 0, 4) and l.shape == (2, 0)


# ---------------------------------------------------------------------------
# Grouped/multi-query attention (chlience notes §5.6: query head h reads
# key/value head floor(h / g), g = H / H_kv, without copying K or V).
# ---------------------------------------------------------------------------

def _gqa_brute(q, k, v, causal, scale):
    """Brute force over [B, H, N, d] with the group written as a contiguous block of
    H / H_kv query heads per key/value head: head h is in group h * H_kv // H."""
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(H):
            grp = (h * H_kv) // H
            o[b, h], lse[b, h] = _brute_force(q[b, h].tolist(), k[b, grp].tolist(), v[b, grp].tolist(),
                                              causal, scale)
    return o, lse


def pin_gqa_brute_force(impl):
    rng = np.random.default_rng(31)
    for H, H_kv in ((6, 1), (6, 2), (6, 3), (6, 6), (4, 2)):
        for causal in (False, True):
            q = rng.standard_normal((2, H, 5, 3))
            k = rng.standard_normal((2, H_kv, 5, 3))
            v = rng.standard_normal((2, H_kv, 5, 3))
            o_ref, l_ref = _gqa_brute(q, k, v, causal, 0.6)
            o, l = impl(q, k, v, causal, 0.6)
            if not (np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)):
                return f"gqa brute force mismatch H={H} H_kv={H_kv} causal={causal}"
    return None


def test_gqa_oracle_pinned():
    assert pin_gqa_brute_force(attention_gqa) is None


def test_gqa_pin_catches_interleaved_mapping():
    """Planted mistake: h % H_kv (interleaved groups) instead of floor(h / g)."""
    def interleaved(q, k, v, causal, scale):
        k2 = np.stack([k[:, h % k.shape[1]] for h in range(q.shape[1])], axis=1)
        v2 = np.stack([v[:, h % v.shape[1]] for h in range(q.shape[1])], axis=1)
        return attention(q, k2, v2, causal, scale)
    assert pin_gqa_brute_force(interleaved) is not None


def test_gqa_closed_forms():
    rng = np.random.default_rng(32)
    # H_kv == H is multi-head attention.
    q, k, v = (rng.standard_normal((1, 4, 7, 5)) for _ in range(3))
    o1, l1 = attention_gqa(q, k, v, True, 0.4)
    o2, l2 = attention(q, k, v, True, 0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # Multi-query: every query head with the same q gives the same row; heads with
    # different q differ.
    qh = rng.standard_normal((7, 5))
    q = np.stack([qh, qh, rng.standard_normal((7, 5))])[None]
    k, v = rng.standard_normal((1, 1, 7, 5)), rng.standard_normal((1, 1, 7, 5))
    o, l = attention_gqa(q, k, v, False, 0.5)
    assert np.array_equal(o[0, 0], o[0, 1]) and not np.allclose(o[0, 0], o[0, 2])
    # Identical V rows inside each group: O of every head of group j equals that row.
    vrow = rng.standard_normal((2, 5))
    v = np.broadcast_to(vrow[None, :, None, :], (1, 2, 7, 5)).copy()
    q, k = rng.standard_normal((1, 6, 7, 5)), rng.standard_normal((1, 2, 7, 5))
    o, _ = attention_gqa(q, k, v, True, 0.5)
    for h in range(6):
        assert np.allclose(o[0, h], vrow[h // 3], atol=1e-14)
    with pytest.raises(ValueError):
        kv_head(0, 6, 4)


def test_varlen_gqa_matches_brute_force():
    rng = np.random.default_rng(33)
    lengths = [3, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, H_kv, d = int(cu[-1]), 4, 2, 3
    q = rng.standard_normal((H, T, d))
    k, v = rng.standard_normal((H_kv, T, d)), rng.standard_normal((H_kv, T, d))
    for causal in (False, True):
        o, l = attention_varlen_gqa(q, k, v, cu, causal, 0.7)
        for s in range(len(lengths)):
            a, b = cu[s], cu[s + 1]
            for h in range(H):
                grp = h * H_kv // H
                ob, lb = _brute_force(q[h, a:b].tolist(), k[grp, a:b].tolist(), v[grp, a:b].tolist(), causal, 0.7)
                assert np.allclose(o[h, a:b], ob, atol=1e-12) and np.allclose(l[h, a:b], lb, atol=1e-12)
