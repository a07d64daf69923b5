"""Pins for the CPU fp64 backward oracle (no GPU needed).

The pages print no numbers for the backward either, so the hand-differentiated oracle
(oracle.attention_backward_head: dV = P^T dO, dP = dO V^T, dS = P o (dP - D),
dQ = scale dS K, dK = scale dS^T Q; chlience notes §5.3, paper-graph-ui §3.4 "The
Backward Pass") is pinned to things that do not share its formulas:

  * central finite differences of the (separately pinned) forward oracle's loss
    sum(dO o O) on tiny inputs;
  * torch's float64 autograd through its own scaled_dot_product_attention;
  * closed forms and invariants: the key-sum of dK vanishes (each row of dS sums to
    zero); the key-sum of dV equals the query-sum of dO (each row of P sums to one);
    equal keys give dQ = 0; dO = 0 gives zero gradients; scale 0 gives uniform
    attention, dQ = dK = 0 and dV_j = sum over allowed i of dO_i / (#keys of row i);
  * grouped-query attention: torch autograd through an explicit head repeat
    (gradients of repeated heads add up, chlience notes §5.6);
  * mutation checks: copies with one planted mistake each (scale dropped from dQ,
    D dropped, D with the wrong sign, P not transposed in dV, mask dropped) must each
    fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import (attention_backward_gqa, attention_backward_head, attention_backward_varlen,
                    attention_head)


def _fd_grads(q, k, v, do, causal, scale, h=1e-6):
    """Central differences of L(Q, K, V) = sum(dO o O(Q, K, V)) with the forward oracle."""
    def loss(qq, kk, vv):
        o, _ = attention_head(qq, kk, vv, causal, scale)
        return float(np.sum(do * o))
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def pin_finite_differences(impl):
    rng = np.random.default_rng(41)
    for n in (1, 2, 4, 6):
        for d in (1, 3):
            for causal in (False, True):
                for mag in (1.0, 2.5):
                    q, k, v = (rng.standard_normal((n, d)) * mag for _ in range(3))
                    do = rng.standard_normal((n, d))
                    ref = _fd_grads(q, k, v, do, causal, 0.8)
                    got = impl(q, k, v, do, causal, 0.8)
                    for name, a, b in zip("qkv", got, ref):
                        if not np.allclose(a, b, rtol=1e-6, atol=1e-7):
                            return f"d{name} vs finite differences n={n} d={d} causal={causal} mag={mag}"
    return None


def pin_torch_autograd(impl):
    rng = np.random.default_rng(42)
    for n, d in ((7, 4), (33, 8), (64, 16)):
        for causal in (False, True):
            # torch's math path masks before scaling, so a negative scale with its causal
            # mask gives NaN: negative scales are compared without the mask only.
            for scale in ((0.35,) if causal else (0.35, -0.2)):
                q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
                tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
                o = torch.nn.functional.scaled_dot_product_attention(
                    tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
                o.backward(torch.tensor(do))
                got = impl(q, k, v, do, causal, scale)
                for name, a, b in zip("qkv", got, (tq.grad, tk.grad, tv.grad)):
                    if not np.allclose(a, b.numpy(), rtol=1e-9, atol=1e-11):
                        return f"d{name} vs torch autograd n={n} causal={causal} scale={scale}"
    return None


def pin_sum_rules(impl):
    rng = np.random.default_rng(43)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((20, 5)) for _ in range(4))
        dq, dk, dv = impl(q, k, v, do, causal, 0.6)
        if not np.allclose(dk.sum(axis=0), 0.0, atol=1e-12):
            return f"key-sum of dK is not zero (causal={causal})"
        if not np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12):
            return f"key-sum of dV differs from query-sum of dO (causal={causal})"
    return None


def pin_closed_forms(impl):
    rng = np.random.default_rng(44)
    n, d = 9, 4
    q, v, do = (rng.standard_normal((n, d)) for _ in range(3))
    k_eq = np.tile(rng.standard_normal((1, d)), (n, 1))
    for causal in (False, True):
        dq, _, _ = impl(q, k_eq, v, do, causal, 0.7)
        if not np.allclose(dq, 0.0, atol=1e-13):
            return "equal keys must give dQ = 0"
        k = rng.standard_normal((n, d))
        g = impl(q, k, v, np.zeros((n, d)), causal, 0.7)
        if any(not np.allclose(x, 0.0, atol=0) for x in g):
            return "dO = 0 must give zero gradients"
        dq, dk, dv = impl(q, k, v, do, causal, 0.0)
        cnt = (np.arange(n) + 1.0) if causal else np.full(n, float(n))
        w = do / cnt[:, None]
        dv_ref = np.array([w[j:].sum(axis=0) if causal else w.sum(axis=0) for j in range(n)])
        if not (np.allclose(dq, 0.0, atol=0) and np.allclose(dk, 0.0, atol=0)
                and np.allclose(dv, dv_ref, atol=1e-13)):
            return f"scale 0 closed form (causal={causal})"
    return None


BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_sum_rules, pin_closed_forms]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pins(pin):
    assert pin(attention_backward_head) is None


def _mutant(kind):
    def impl(q, k, v, do, causal, scale):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        n = q.shape[0]
        s = scale * (q @ k.T)
        if causal and kind != "no_mask":
            s[np.triu_indices(n, k=1)] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v
        dv = (p @ do) if kind == "dv_no_transpose" else (p.T @ do)
        dp = do @ v.T
        dvec = np.sum(do * o, axis=1, keepdims=True)
        if kind == "no_d":
            ds = p * dp
        elif kind == "d_sign":
            ds = p * (dp + dvec)
        else:
            ds = p * (dp - dvec)
        dq = (ds @ k) if kind == "no_scale_dq" else scale * (ds @ k)
        dk = scale * (ds.T @ q)
        return dq, dk, dv
    return impl


@pytest.mark.parametrize("kind", ["no_scale_dq", "no_d", "d_sign", "dv_no_transpose", "no_mask"])
def test_backward_pins_catch_planted_mistakes(kind):
    impl = _mutant(kind)
    assert any(pin(impl) is not None for pin in BWD_PINS), kind


def test_backward_gqa_vs_autograd_repeat():
    rng = np.random.default_rng(45)
    B, H, H_kv, N, d = 2, 6, 2, 11, 4
    q, do = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    k, v = rng.standard_normal((B, H_kv, N, d)), rng.standard_normal((B, H_kv, N, d))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        g = H // H_kv
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), is_causal=causal, scale=0.45)
        o.backward(torch.tensor(do))
        dq, dk, dv = attention_backward_gqa(q, k, v, do, causal, 0.45)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_backward_varlen_matches_per_sequence():
    rng = np.random.default_rng(46)
    lengths = [3, 1, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    H, H_kv, T, d = 4, 2, int(cu[-1]), 3
    q, do = rng.standard_normal((H, T, d)), rng.standard_normal((H, T, d))
    k, v = rng.standard_normal((H_kv, T, d)), rng.standard_normal((H_kv, T, d))
    for causal in (False, True):
        dq, dk, dv = attention_backward_varlen(q, k, v, do, cu, causal, 0.5)
        for s in range(len(lengths)):
            a, b = cu[s], cu[s + 1]
            gq, gk, gv = attention_backward_gqa(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b],
                                                do[None, :, a:b], causal, 0.5)
            assert np.allclose(dq[:, a:b], gq[0], atol=1e-13)
            assert np.allclose(dk[:, a:b], gk[0], atol=1e-13)
            assert np.allclose(dv[:, a:b], gv[0], atol=1e-13)
