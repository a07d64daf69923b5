"""The library's calls captured in a HIP graph and replayed.

Every entry point enqueues only kernel launches on the caller's stream (no allocation, no
memset, no host synchronisation), so a caller may capture it in a graph and replay it.
Each test captures one call with fixed device buffers. It then replays the graph several
times, with the program's own eager work between replays: new inputs copied into the
captured input buffers and the outputs overwritten with NaN. Every replay must reproduce,
bit for bit, the eager call on the same inputs. The kernels use no atomics in their
arithmetic, so equal inputs give equal bits. (Under capture, fa2_fwd_varlen and
fa2_bwd_varlen launch their one-workgroup-per-block kernels in place of the persistent
forms.)
"""
import pytest
import torch

import exact_softmax_attention_amd as fa2
from synthetic import make_qkv, make_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _capture(fn):
    """Warm the call up on a side stream, then capture it (torch's documented pattern)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, inputs, input_sets, outputs, refs, tag):
    """Replay g REPLAYS times, alternating between the input sets."""
    for rep in range(REPLAYS):
        which = rep % len(input_sets)
        for buf, val in zip(inputs, input_sets[which]):
            buf.copy_(val)
        for out in outputs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[case] {tag} replay {rep} inputs {which}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for name, out, ref in zip(("0", "1", "2", "3"), outputs, refs[which]):
            assert torch.equal(out, ref), f"{tag}: replay {rep} output {name} differs from the eager call"


def _two_qkv_sets(B, H, N, d, seed, H_kv=None):
    a = [t.to(DEV) for t in make_qkv(B, H, N, d, seed, H_kv=H_kv)]
    b = [t.to(DEV) for t in make_qkv(B, H, N, d, seed + 1, H_kv=H_kv)]
    return a, b


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_graph(d, causal):
    sets = _two_qkv_sets(2, 4, 1000, d, seed=900 + d)
    q, k, v = [t.clone() for t in sets[0]]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    refs = []
    for s in sets:
        ro, rl = fa2.fwd(*s, causal=causal)
        refs.append((ro.clone(), rl.clone()))
    g = _capture(lambda: fa2.fwd(q, k, v, causal=causal, out=o, lse=lse))
    _replay_and_check(g, (q, k, v), sets, (o, lse), refs, f"fwd d{d} causal={causal}")


def test_varlen_forward_graph():
    H, d = 4, 128
    lengths = [300, 1, 777, 64]
    sets = []
    for seed in (910, 911):
        q, k, v, cu, _ = make_varlen(H, d, seed, lengths=lengths)
        sets.append((q.to(DEV), k.to(DEV), v.to(DEV)))
    cu = cu.to(DEV)
    q, k, v = [t.clone() for t in sets[0]]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    refs = []
    for s in sets:
        ro, rl = fa2.fwd_varlen(*s, cu, max(lengths), causal=True)
        refs.append((ro.clone(), rl.clone()))
    g = _capture(lambda: fa2.fwd_varlen(q, k, v, cu, max(lengths), causal=True, out=o, lse=lse))
    _replay_and_check(g, (q, k, v), sets, (o, lse), refs, "varlen fwd")


@pytest.mark.parametrize("h_kv", [4, 2])
def test_backward_graph(h_kv):
    B, H, N, d = 1, 4, 700, 128
    sets = []
    for seed in (920, 921):
        q, k, v = [t.to(DEV) for t in make_qkv(B, H, N, d, seed, H_kv=h_kv)]
        o, lse = fa2.fwd_gqa(q, k, v, causal=True)
        gen = torch.Generator().manual_seed(seed)
        dout = torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(DEV)
        sets.append((q, k, v, o.clone(), lse.clone(), dout))
    bufs = [t.clone() for t in sets[0]]
    dq, dk, dv = torch.empty_like(bufs[0]), torch.empty_like(bufs[1]), torch.empty_like(bufs[2])
    delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    refs = []
    for s in sets:
        rq, rk, rv = fa2.bwd(*s, causal=True)
        refs.append((rq.clone(), rk.clone(), rv.clone()))
    g = _capture(lambda: fa2.bwd(*bufs, causal=True, dq=dq, dk=dk, dv=dv, delta=delta))
    _replay_and_check(g, bufs, sets, (dq, dk, dv), refs, f"bwd H_kv={h_kv}")


def test_split_kv_graph():
    B, H, N_q, N_k, d, S = 1, 4, 200, 2000, 128, 4
    sets = []
    for seed in (930, 931):
        q = make_qkv(B, H, N_q, d, seed)[0].to(DEV)
        _, k, v = make_qkv(B, H, N_k, d, seed + 100)
        sets.append((q, k.to(DEV), v.to(DEV)))
    q, k, v = [t.clone() for t in sets[0]]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    o_parts = torch.empty((S, B, H, N_q, d), dtype=torch.bfloat16, device=DEV)
    l_parts = torch.empty((S, B, H, N_q), dtype=torch.float32, device=DEV)
    refs = []
    for s in sets:
        ro, rl = fa2.fwd_splitkv(*s, S, causal=True, diag=N_k - N_q)
        refs.append((ro.clone(), rl.clone()))
    g = _capture(lambda: fa2.fwd_splitkv(q, k, v, S, causal=True, diag=N_k - N_q, out=o, lse=lse,
                                         o_parts=o_parts, lse_parts=l_parts))
    _replay_and_check(g, (q, k, v), sets, (o, lse), refs, "split-kv")
