"""Pins for the oracle's key/value-chunk attention and LSE merge (no GPU needed).

oracle.attention_chunk_head (attention of a query block over one key chunk, with the causal
diagonal offset diag: query i may attend key j iff j <= i + diag) and oracle.lse_merge
(LSE = log sum exp LSE_s, O = sum exp(LSE_s - LSE) O_s; llm-infra-atlas "FlashAttention"
§5 and its §0 reading table) are pinned to:

  * the partition identity: chunks of a key sequence, merged, give exactly the full
    attention of the separately pinned oracle (causal and not, empty chunks, chunks that a
    row cannot see);
  * bottom-right alignment: the last N_q queries of a causal sequence over all N_k keys are
    the chunk call with diag = N_k - N_q;
  * brute force on tiny inputs with scalar loops;
  * merge closed forms: one part is the identity, the order of parts does not matter, two
    equal parts keep O and add ln 2 to LSE, all -inf gives O = 0 and LSE = -inf, and huge
    LSE values (1e4) do not overflow;
  * mutation checks: a merge without the max subtraction, one without normalisation, and a
    chunk mask with diag of the wrong sign must each fail.
"""
import math

import numpy as np
import pytest

from oracle import attention_chunk, attention_chunk_head, attention_head, lse_merge


def _split_merge(chunk_fn, merge_fn, q, k, v, causal, scale, cuts):
    bounds = [0, *cuts, k.shape[0]]
    os, ls = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = chunk_fn(q, k[a:b], v[a:b], causal, -a, scale)
        os.append(o)
        ls.append(l)
    return merge_fn(np.stack(os), np.stack(ls))


def pin_partition(chunk_fn, merge_fn):
    rng = np.random.default_rng(51)
    for causal in (False, True):
        for cuts in ([20], [7, 7, 30], [1, 39], [13, 26]):
            q, k, v = (rng.standard_normal((40, 6)) * 1.5 for _ in range(3))
            o, l = _split_merge(chunk_fn, merge_fn, q, k, v, causal, 0.5, cuts)
            o_ref, l_ref = attention_head(q, k, v, causal, 0.5)
            if not (np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)):
                return f"chunks {cuts} merged != full attention (causal={causal})"
    return None


def pin_bottom_right(chunk_fn):
    rng = np.random.default_rng(52)
    for nq in (1, 5, 17):
        q, k, v = (rng.standard_normal((30, 4)) for _ in range(3))
        o_ref, l_ref = attention_head(q, k, v, True, 0.7)
        o, l = chunk_fn(q[30 - nq:], k, v, True, 30 - nq, 0.7)
        if not (np.allclose(o, o_ref[30 - nq:], atol=1e-13) and np.allclose(l, l_ref[30 - nq:], atol=1e-13)):
            return f"bottom-right alignment n_q={nq}"
    return None


def pin_chunk_brute_force(chunk_fn):
    rng = np.random.default_rng(53)
    for nq, nk in ((1, 1), (3, 5), (5, 3), (4, 4)):
        for diag in (-2, 0, 1, 3):
            q, k, v = rng.standard_normal((nq, 3)), rng.standard_normal((nk, 3)), rng.standard_normal((nk, 2))
            o, l = chunk_fn(q, k, v, True, diag, 0.9)
            for i in range(nq):
                js = [j for j in range(nk) if j <= i + diag]
                if not js:
                    if not (np.all(o[i] == 0) and l[i] == -np.inf):
                        return f"row without keys n_q={nq} n_k={nk} diag={diag}"
                    continue
                w = [math.exp(0.9 * math.fsum(q[i, t] * k[j, t] for t in range(3))) for j in js]
                z = math.fsum(w)
                oi = [math.fsum(wj * v[j, c] for wj, j in zip(w, js)) / z for c in range(2)]
                if not (np.allclose(o[i], oi, atol=1e-12) and abs(l[i] - math.log(z)) < 1e-12):
                    return f"brute force n_q={nq} n_k={nk} diag={diag}"
    return None


def pin_merge_closed_forms(merge_fn):
    rng = np.random.default_rng(54)
    o1, l1 = rng.standard_normal((7, 4)), rng.standard_normal(7) * 3
    o, l = merge_fn(o1[None], l1[None])
    if not (np.allclose(o, o1, atol=1e-15) and np.allclose(l, l1, atol=1e-15)):
        return "one part must be the identity"
    o2, l2 = rng.standard_normal((7, 4)), rng.standard_normal(7) * 3
    a = merge_fn(np.stack([o1, o2]), np.stack([l1, l2]))
    b = merge_fn(np.stack([o2, o1]), np.stack([l2, l1]))
    if not (np.allclose(a[0], b[0], atol=1e-15) and np.allclose(a[1], b[1], atol=1e-15)):
        return "order of parts changed the result"
    o, l = merge_fn(np.stack([o1, o1]), np.stack([l1, l1]))
    if not (np.allclose(o, o1, atol=1e-14) and np.allclose(l, l1 + math.log(2), atol=1e-14)):
        return "two equal parts must keep O and add ln 2"
    o, l = merge_fn(np.stack([o1, o2]), np.full((2, 7), -np.inf))
    if not (np.all(o == 0) and np.all(l == -np.inf)):
        return "all -inf must give O = 0, LSE = -inf"
    big = np.stack([l1 + 1e4, l2 + 1e4])
    o, l = merge_fn(np.stack([o1, o2]), big)
    if not (np.all(np.isfinite(o)) and np.allclose(o, a[0], atol=1e-12) and np.allclose(l, a[1] + 1e4, atol=1e-9)):
        return "large LSE values"
    return None


def test_chunk_and_merge_pinned():
    assert pin_partition(attention_chunk_head, lse_merge) is None
    assert pin_bottom_right(attention_chunk_head) is None
    assert pin_chunk_brute_force(attention_chunk_head) is None
    assert pin_merge_closed_forms(lse_merge) is None


def _merge_no_max(o_parts, lse_parts):
    w = np.exp(lse_parts)
    z = w.sum(axis=0)
    return np.sum((w / z)[..., None] * o_parts, axis=0), np.log(z)


def _merge_unnormalised(o_parts, lse_parts):
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    return np.sum(w[..., None] * o_parts, axis=0), m + np.log(w.sum(axis=0))


def _chunk_wrong_diag(q, k, v, causal, diag, scale):
    return attention_chunk_head(q, k, v, causal, -diag, scale)


@pytest.mark.parametrize("mutant", ["merge_no_max", "merge_unnormalised", "chunk_wrong_diag"])
def test_merge_pins_catch_planted_mistakes(mutant):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        if mutant == "merge_no_max":
            assert pin_merge_closed_forms(_merge_no_max) is not None
        elif mutant == "merge_unnormalised":
            assert pin_partition(attention_chunk_head, _merge_unnormalised) is not None
        else:
            assert (pin_partition(_chunk_wrong_diag, lse_merge) is not None
                    or pin_bottom_right(_chunk_wrong_diag) is not None)


def test_chunk_batched_and_gqa():
    rng = np.random.default_rng(55)
    q = rng.standard_normal((2, 4, 9, 5))
    k, v = rng.standard_normal((2, 2, 13, 5)), rng.standard_normal((2, 2, 13, 5))
    o, l = attention_chunk(q, k, v, True, 4, 0.3)
    for b in range(2):
        for h in range(4):
            oh, lh = attention_chunk_head(q[b, h], k[b, h // 2], v[b, h // 2], True, 4, 0.3)
            assert np.array_equal(o[b, h], oh) and np.array_equal(l[b, h], lh)
    o, l = attention_chunk(q, k[:, :, :0], v[:, :, :0], False, 0, 0.3)
    assert np.all(o == 0) and np.all(l == -np.inf)
