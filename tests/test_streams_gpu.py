"""Calls on two streams at once: the library keeps no state between calls (the header's
reentrancy statement), so work enqueued on two streams that may run concurrently gives
the same bits as the same calls made one after the other on one stream."""
import pytest
import torch

import exact_softmax_attention_amd as fa2
from synthetic import make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_two_streams_match_serial_calls():
    a = [t.to(DEV) for t in make_qkv(2, 8, 1500, 128, seed=960)]
    b = [t.to(DEV) for t in make_qkv(1, 4, 3000, 64, seed=961, H_kv=2)]
    gen = torch.Generator().manual_seed(962)
    dout_a = torch.randn(a[0].shape, generator=gen).to(torch.bfloat16).to(DEV)
    # serial references on the current stream
    oa_ref, la_ref = fa2.fwd(*a, causal=True)
    ob_ref, lb_ref = fa2.fwd_gqa(*b, causal=False)
    ga_ref = fa2.bwd(*a, oa_ref, la_ref, dout_a, causal=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()     # default priority
    for rep in range(3):
        print(f"[case] two streams rep {rep}", flush=True)
        with torch.cuda.stream(s1):
            oa, la = fa2.fwd(*a, causal=True)
            ga = fa2.bwd(*a, oa, la, dout_a, causal=True)
        with torch.cuda.stream(s2):
            ob, lb = fa2.fwd_gqa(*b, causal=False)
        torch.cuda.synchronize()
        assert torch.equal(oa, oa_ref) and torch.equal(la, la_ref)
        assert torch.equal(ob, ob_ref) and torch.equal(lb, lb_ref)
        for g, r in zip(ga, ga_ref):
            assert torch.equal(g, r)
