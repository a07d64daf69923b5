"""The persistent kernels: a fixed grid of workgroups taking blocks from a work queue. The
forward's runs in fa2_fwd_varlen at head dimensions 72..128; the backward's dQ and dK/dV
forms run in fa2_bwd_varlen at head dimensions 72..256.

Their blocks are those of the ordinary kernels, so every output must match those kernels
bit for bit, whichever workgroup takes a block. The forward is compared with variant 0
(the ordinary kernel of the same tiles). The backward is compared with the same call
captured in a graph, since under capture fa2_bwd_varlen launches the ordinary kernels. The
queue counters come from a static pool of sets that each launch returns to zero. The tests
therefore run more launches than the pool has sets, so every set is reused, and interleave
launches on several streams. Outputs are prefilled with NaN so that a block the queue
skipped shows up. Parity against the oracle runs here as well, on batches with empty,
one-token and tile-edge sequences.
"""
import math

import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_backward_varlen, attention_varlen
from synthetic import make_qkv, make_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
POOL_SETS = 1024          # counter sets in the library's pool (header of fa2_fwd_varlen)


def _persist_index():
    names = [fa2.variant_name(128, i) for i in range(fa2.num_variants(128))]
    return names.index("d128_w8_bc64_persist")


def _varlen_on_device(H, d, seed, lengths):
    q, k, v, cu, lengths = make_varlen(H, d, seed, lengths=lengths)
    return (q, k, v, cu, lengths), (q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV))


def _nan_outputs(q):
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [96, 128])
def test_default_varlen_parity_and_bitwise(d, causal):
    # Many short sequences and a long one: most row blocks of the grid the ordinary kernel
    # launches lie past the end of their sequence.
    lengths = [0, 1, 2, 63, 64, 65, 255, 256, 257, 0, 3000, 7, 128, 129, 1, 0, 511, 512, 1024, 33]
    (q, k, v, cu, lengths), (qd, kd, vd, cud) = _varlen_on_device(4, d, 1300 + d + int(causal), lengths)
    scale = 1.0 / math.sqrt(d)
    maxlen = max(lengths) + 5
    o, lse = _nan_outputs(qd)
    print(f"[case] persistent varlen d{d} causal={causal}", flush=True)
    fa2.fwd_varlen(qd, kd, vd, cud, maxlen, causal=causal, scale=scale, out=o, lse=lse)
    o0, l0 = fa2.fwd_varlen(qd, kd, vd, cud, maxlen, causal=causal, scale=scale, variant=0)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0), "default varlen differs from variant 0"
    o_ref, l_ref = attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(), cu.numpy(),
                                    causal, scale)
    err = np.abs(o.float().cpu().double().numpy() - o_ref)
    lerr = np.abs(lse.cpu().double().numpy() - l_ref)
    print(f"[parity] persistent d{d} causal={causal}: O max {err.max():.3e} mean {err.mean():.3e} "
          f"| LSE max {lerr.max():.3e}", flush=True)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX


def test_pool_reuse_many_launches():
    """More launches than the pool has sets, alternating a batch of many row blocks with one
    smaller than the grid: every set is taken again after its launch returned it to zero."""
    big, bigd = _varlen_on_device(2, 128, 1320, [4096, 17, 900, 0, 2048, 1])
    small, smalld = _varlen_on_device(1, 128, 1321, [5, 300])
    refs = []
    for (_, _, _, _, lengths), (qd, kd, vd, cud) in ((big, bigd), (small, smalld)):
        refs.append(fa2.fwd_varlen(qd, kd, vd, cud, max(lengths), causal=True, variant=0))
    outs = [_nan_outputs(bigd[0]), _nan_outputs(smalld[0])]
    torch.cuda.synchronize()
    calls = POOL_SETS + POOL_SETS // 2 + 7
    for i in range(calls):
        which = i % 2
        (_, _, _, _, lengths), (qd, kd, vd, cud) = (big, bigd) if which == 0 else (small, smalld)
        o, lse = outs[which]
        if i % 64 == which:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        fa2.fwd_varlen(qd, kd, vd, cud, max(lengths), causal=True, out=o, lse=lse)
        if i % 64 == which:
            torch.cuda.synchronize()
            ro, rl = refs[which]
            assert torch.equal(o, ro) and torch.equal(lse, rl), f"call {i} differs from variant 0"
        if i % 256 == 0:
            print(f"[case] pool reuse call {i} of {calls}", flush=True)
    torch.cuda.synchronize()
    for (o, lse), (ro, rl) in zip(outs, refs):
        assert torch.equal(o, ro) and torch.equal(lse, rl)


def test_streams_interleaved():
    """Persistent launches on four streams at once (each with its own counter set) give the
    bits of the same calls made one by one."""
    cases = []
    for j, lengths in enumerate(([1000, 3, 2500], [64] * 40, [1, 2, 3, 4, 4000], [700, 700, 0, 1500])):
        host, dev = _varlen_on_device(2, 128, 1330 + j, lengths)
        ref = fa2.fwd_varlen(*dev[:3], dev[3], max(host[4]), causal=bool(j % 2), variant=0)
        cases.append((host[4], dev, ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]     # default priority
    for rep in range(4):
        print(f"[case] four streams rep {rep}", flush=True)
        outs = []
        for j, ((lengths, dev, _), s) in enumerate(zip(cases, streams)):
            o, lse = _nan_outputs(dev[0])
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(3):
                    fa2.fwd_varlen(*dev[:3], dev[3], max(lengths), causal=bool(j % 2), out=o, lse=lse)
            outs.append((o, lse))
        torch.cuda.synchronize()
        for (o, lse), (_, _, (ro, rl)) in zip(outs, cases):
            assert torch.equal(o, ro) and torch.equal(lse, rl)


@pytest.mark.parametrize("causal", [False, True])
def test_fixed_length_persistent_variant(causal):
    """The persistent variant through the fixed-length and split-KV entry points."""
    p = _persist_index()
    q, k, v = [t.to(DEV) for t in make_qkv(2, 5, 1111, 128, seed=1340 + int(causal))]
    o0, l0 = fa2.fwd(q, k, v, causal=causal, variant=0)
    o1, l1 = fa2.fwd(q, k, v, causal=causal, variant=p)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    # One piece runs the persistent kernel, three the one-block-per-workgroup one; a query
    # chunk at the end of the keys (diag) shifts the causal diagonal.
    for splits, diag in ((1, 0), (3, 0), (1, 400), (3, 400)):
        print(f"[case] persistent split-KV splits={splits} diag={diag} causal={causal}", flush=True)
        qc = q[:, :, -300:].contiguous() if diag else q
        s0 = fa2.fwd_splitkv(qc, k, v, num_splits=splits, causal=causal, diag=diag, variant=0)
        s1 = fa2.fwd_splitkv(qc, k, v, num_splits=splits, causal=causal, diag=diag, variant=p)
        torch.cuda.synchronize()
        for a, b in zip(s0, s1):
            assert torch.equal(a, b), (splits, diag)


def _bwd_varlen_case(H, d, seed, lengths, causal):
    (q, k, v, cu, lengths), (qd, kd, vd, cud) = _varlen_on_device(H, d, seed, lengths)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.fwd_varlen(qd, kd, vd, cud, max(lengths), causal=causal, scale=scale)
    gen = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(q.shape, generator=gen).to(torch.bfloat16)
    return (q, k, v, cu, lengths, dout), (qd, kd, vd, o, lse, dout.to(DEV), cud), scale


def _nan_grads(qd, kd, vd, lse):
    return (torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")),
            torch.full_like(vd, float("nan")), torch.full_like(lse, float("nan")))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 256])
def test_bwd_varlen_persistent_matches_ordinary(d, causal):
    """Eager fa2_bwd_varlen (persistent kernels) against the same call captured in a graph
    (ordinary kernels): bitwise equal; and against the oracle's backward."""
    lengths = [0, 1, 2, 127, 128, 129, 0, 700, 5, 1000, 64, 1]
    host, dev, scale = _bwd_varlen_case(2, d, 1350 + d + int(causal), lengths, causal)
    qd, kd, vd, o, lse, dout, cud = dev
    maxlen = max(host[4])
    dq, dk, dv, delta = _nan_grads(qd, kd, vd, lse)
    print(f"[case] persistent bwd varlen d{d} causal={causal}", flush=True)
    fa2.bwd_varlen(qd, kd, vd, o, lse, dout, cud, maxlen, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,
                   delta=delta)
    torch.cuda.synchronize()
    cq, ck, cv, cdelta = _nan_grads(qd, kd, vd, lse)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fa2.bwd_varlen(qd, kd, vd, o, lse, dout, cud, maxlen, causal=causal, scale=scale, dq=cq, dk=ck, dv=cv,
                       delta=cdelta)
    torch.cuda.synchronize()
    for rep in range(2):
        for t in (cq, ck, cv, cdelta):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in ((dq, cq, "dq"), (dk, ck, "dk"), (dv, cv, "dv"), (delta, cdelta, "delta")):
            assert torch.equal(a, b), f"{name} of the persistent kernels differs from the ordinary ones (replay {rep})"
    q, k, v, cu, lengths, dout_h = host
    ref = attention_backward_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                    dout_h.double().numpy(), cu.numpy(), causal, scale)
    # Gradient tolerance as in the backward parity tests: relative to the largest reference
    # entry, max 2e-2 and mean 2e-3 (a few bf16 roundings of the summed terms).
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        err = np.abs(got.float().cpu().double().numpy() - want)
        top = float(np.abs(want).max())
        print(f"[parity] persistent bwd d{d} causal={causal} {name}: max {err.max() / top:.2e} "
              f"mean {err.mean() / top:.2e} of max|ref| {top:.3e}", flush=True)
        assert np.all(np.isfinite(err)) and err.max() <= 2e-2 * top and err.mean() <= 2e-3 * top


def test_bwd_pool_reuse_and_streams():
    """Backward varlen calls (two counter sets each) past the pool's size, then on three
    streams at once: every result equals the first call's."""
    cases = []
    for j, lengths in enumerate(([900, 3, 0, 1500], [64] * 12, [1, 2000])):
        host, dev, scale = _bwd_varlen_case(2, 128, 1370 + j, lengths, causal=bool(j % 2))
        qd, kd, vd, o, lse, dout, cud = dev
        ref = fa2.bwd_varlen(qd, kd, vd, o, lse, dout, cud, max(host[4]), causal=bool(j % 2), scale=scale)
        cases.append((max(host[4]), dev, scale, bool(j % 2), [r.clone() for r in ref]))
    torch.cuda.synchronize()
    calls = POOL_SETS // 2 + 40
    for i in range(calls):
        maxlen, (qd, kd, vd, o, lse, dout, cud), scale, causal, ref = cases[i % 2]
        out = fa2.bwd_varlen(qd, kd, vd, o, lse, dout, cud, maxlen, causal=causal, scale=scale)
        if i % 50 == 0 or i >= calls - 2:
            torch.cuda.synchronize()
            for a, b in zip(out, ref):
                assert torch.equal(a, b), f"call {i}"
        if i % 200 == 0:
            print(f"[case] bwd pool reuse call {i} of {calls}", flush=True)
    streams = [torch.cuda.Stream() for _ in cases]     # default priority
    for rep in range(3):
        print(f"[case] bwd three streams rep {rep}", flush=True)
        outs = []
        for (maxlen, (qd, kd, vd, o, lse, dout, cud), scale, causal, _), st in zip(cases, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(fa2.bwd_varlen(qd, kd, vd, o, lse, dout, cud, maxlen, causal=causal, scale=scale))
        torch.cuda.synchronize()
        for out, case in zip(outs, cases):
            for a, b in zip(out, case[4]):
                assert torch.equal(a, b)
