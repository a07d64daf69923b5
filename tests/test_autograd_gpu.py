"""The autograd wrappers: gradients through torch's autograd equal the direct backward calls.

``fa2.attention`` and ``fa2.attention_varlen`` only route arguments between the forward and
backward entry points, whose numerics the parity tests check against the oracle. So these
tests compare, bit for bit, the wrapper's O and LSE with the direct forward call, and
q.grad, k.grad and v.grad with the direct backward call on the same upstream gradient. That
pins the wiring (saved tensors, argument order, the gradient order returned to autograd),
including a non-contiguous upstream gradient. One case also goes to the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_backward_gqa
from synthetic import make_qkv, make_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _leaf(t):
    return t.to(DEV).requires_grad_(True)


@pytest.mark.parametrize("h_kv", [4, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_grads_equal_direct_calls(causal, h_kv):
    B, H, N, d = 2, 4, 300, 128
    q0, k0, v0 = make_qkv(B, H, N, d, seed=950 + h_kv, H_kv=h_kv)
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    gen = torch.Generator().manual_seed(951)
    dout = torch.randn((B, H, N, d), generator=gen).to(torch.bfloat16).to(DEV)
    print(f"[case] autograd causal={causal} H_kv={h_kv}", flush=True)
    o, lse = fa2.attention(q, k, v, causal=causal, return_lse=True)
    o.backward(dout)
    torch.cuda.synchronize()
    qd, kd, vd = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    o_ref, l_ref = fa2.fwd_gqa(qd, kd, vd, causal=causal)
    dq, dk, dv = fa2.bwd(qd, kd, vd, o_ref, l_ref, dout, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref) and torch.equal(lse, l_ref)
    assert not lse.requires_grad
    for name, got, ref in (("dq", q.grad, dq), ("dk", k.grad, dk), ("dv", v.grad, dv)):
        assert torch.equal(got, ref), f"{name} through autograd differs from the direct call"


def test_noncontiguous_upstream_gradient():
    B, H, N, d = 1, 2, 200, 64
    q0, k0, v0 = make_qkv(B, H, N, d, seed=952)
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    gen = torch.Generator().manual_seed(953)
    g_t = torch.randn((B, N, H, d), generator=gen).to(torch.bfloat16).to(DEV)   # [B, N, H, d]
    o = fa2.attention(q, k, v, causal=True, scale=0.1)
    (o.transpose(1, 2).float() * g_t.float()).sum().backward()   # dO = g_t^T, a strided view
    torch.cuda.synchronize()
    qd, kd, vd = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    o_ref, l_ref = fa2.fwd(qd, kd, vd, causal=True, scale=0.1)
    dq, dk, dv = fa2.bwd(qd, kd, vd, o_ref, l_ref, g_t.transpose(1, 2).contiguous(), causal=True, scale=0.1)
    torch.cuda.synchronize()
    for got, ref in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(got, ref)


def test_attention_varlen_grads_equal_direct_calls():
    H, H_kv, d = 4, 2, 64
    lengths = [100, 1, 257, 64]
    q0, k0, v0, cu, _ = make_varlen(H, d, seed=954, lengths=lengths, H_kv=H_kv)
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    cud = cu.to(DEV)
    gen = torch.Generator().manual_seed(955)
    dout = torch.randn(q0.shape, generator=gen).to(torch.bfloat16).to(DEV)
    o = fa2.attention_varlen(q, k, v, cud, max(lengths), causal=True)
    o.backward(dout)
    torch.cuda.synchronize()
    qd, kd, vd = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    o_ref, l_ref = fa2.fwd_varlen_gqa(qd, kd, vd, cud, max(lengths), causal=True)
    dq, dk, dv = fa2.bwd_varlen(qd, kd, vd, o_ref, l_ref, dout, cud, max(lengths), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for got, ref in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(got, ref)


def test_attention_grads_against_the_oracle():
    """The wrapper's gradients against the oracle, with the backward parity tests' tolerance
    (error relative to the largest reference entry: max 2e-2, mean 2e-3)."""
    B, H, H_kv, N, d = 1, 4, 2, 150, 128
    q0, k0, v0 = make_qkv(B, H, N, d, seed=956, H_kv=H_kv)
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    gen = torch.Generator().manual_seed(957)
    dout0 = torch.randn((B, H, N, d), generator=gen).to(torch.bfloat16)
    fa2.attention(q, k, v, causal=True).backward(dout0.to(DEV))
    torch.cuda.synchronize()
    refs = attention_backward_gqa(q0.double().numpy(), k0.double().numpy(), v0.double().numpy(),
                                  dout0.double().numpy(), True, 1.0 / math.sqrt(d))
    for name, got, ref in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), refs):
        err = np.abs(got.float().cpu().double().numpy() - ref)
        top = float(np.abs(ref).max())
        print(f"[parity] autograd {name}: max {err.max() / top:.2e} mean {err.mean() / top:.2e} of max|ref|",
              flush=True)
        assert err.max() <= 2e-2 * top and err.mean() <= 2e-3 * top, name
