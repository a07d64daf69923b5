"""GPU parity for the backward with query-head splits (fa2_bwd_ws) against the fp64 oracle.

With grouped- or multi-query heads the Python ``bwd`` calls fa2_bwd_ws, which spreads each
group's query heads over several dK/dV workgroups and adds their fp32 partials in a third
kernel; ``split=False`` calls fa2_bwd (one workgroup per key/value head and key block). Both
are compared with oracle.attention_backward_gqa / attention_backward_head (the gradient of a
shared key/value head is the sum over its query heads), with the tolerance derived in
test_parity_bwd_gpu.py: max error <= 2e-2 and mean error <= 2e-3 of max|reference|.
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_backward_gqa, attention_backward_head
from synthetic import make_qkv

pytestmark = pytest.mark.gpu

G_MAX, G_MEAN = 2e-2, 2e-3
DEV = "cuda:0"


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _dout(shape, seed):
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def _check_grad(g, ref, tag):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{tag}: non-finite gradient"
    scale = float(np.abs(ref).max(initial=0.0))
    err = np.abs(g - ref)
    rel_mx = float(err.max(initial=0.0)) / scale
    rel_mean = float(err.mean()) / scale
    print(f"[parity] {tag}: max {rel_mx:.2e} mean {rel_mean:.2e} of max|ref| {scale:.3e}", flush=True)
    assert rel_mx <= G_MAX and rel_mean <= G_MEAN, tag


def _grads(q, k, v, do, causal, scale, split):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa2.fwd_gqa(qd, kd, vd, causal=causal, scale=scale)
    out = fa2.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, split=split)
    torch.cuda.synchronize()
    return out


def _ws_bytes(q, k, causal):
    B, H, N, d = q.shape
    return fa2.load_library().fa2_bwd_workspace_bytes(B, H, k.shape[1], N, d, int(causal))


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("H,H_kv,N", [(8, 2, 300), (8, 1, 129), (6, 3, 1000), (16, 2, 64)])
def test_split_small(d, H, H_kv, N):
    q, k, v = make_qkv(2, H, N, d, seed=500 + d + N + H_kv, H_kv=H_kv)
    do = _dout(q.shape, 600 + d + N)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        assert _ws_bytes(q, k, causal) > 0, "shape does not exercise the split"
        tag = f"bwd split d{d} {H}/{H_kv} N{N} causal={causal}"
        print(f"[case] {tag}", flush=True)
        rq, rk, rv = attention_backward_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                            do.double().numpy(), causal, scale)
        for split in (True, False):
            dq, dk, dv = _grads(q, k, v, do, causal, scale, split)
            t = tag + (" ws" if split else " plain")
            _check_grad(_f64(dq), rq, t + " dQ")
            _check_grad(_f64(dk), rk, t + " dK")
            _check_grad(_f64(dv), rv, t + " dV")


def test_split_long_gqa():
    """B=1 H=16 H_kv=2 N=16384 d=128 causal (eight splits of one query head per key/value
    head): dK and dV of key/value head 1 over every element against the oracle's sum over
    query heads 8..15, dQ of query head 13."""
    B, H, H_kv, N, d = 1, 16, 2, 16384, 128
    q, k, v = make_qkv(B, H, N, d, seed=510, H_kv=H_kv)
    do = _dout(q.shape, 610)
    scale = 1.0 / np.sqrt(d)
    assert _ws_bytes(q, k, True) == 8 * 2 * B * H_kv * N * d * 4
    print("[case] bwd split long B1 H16/2 N16384 d128 causal", flush=True)
    dq, dk, dv = _grads(q, k, v, do, True, scale, True)
    hk = 1
    sk = np.zeros((N, d))
    sv = np.zeros((N, d))
    for h in range(hk * 8, hk * 8 + 8):
        rq, rk, rv = attention_backward_head(q[0, h].double().numpy(), k[0, hk].double().numpy(),
                                             v[0, hk].double().numpy(), do[0, h].double().numpy(), True, scale)
        sk += rk
        sv += rv
        if h == 13:
            _check_grad(_f64(dq[0, h]), rq, "bwd split long dQ h13")
        del rq, rk, rv
    _check_grad(_f64(dk[0, hk]), sk, "bwd split long dK hk1")
    _check_grad(_f64(dv[0, hk]), sv, "bwd split long dV hk1")


def test_split_mqa_all_heads():
    """Multi-query: B=1 H=16 H_kv=1 N=4096 d=128 causal (16 splits of one query head), every
    element of dQ, dK and dV."""
    q, k, v = make_qkv(1, 16, 4096, 128, seed=520, H_kv=1)
    do = _dout(q.shape, 620)
    scale = 1.0 / np.sqrt(128)
    assert _ws_bytes(q, k, True) == 16 * 2 * 1 * 1 * 4096 * 128 * 4
    print("[case] bwd split mqa B1 H16/1 N4096 d128 causal", flush=True)
    dq, dk, dv = _grads(q, k, v, do, True, scale, True)
    rq, rk, rv = attention_backward_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        do.double().numpy(), True, scale)
    _check_grad(_f64(dq), rq, "bwd split mqa dQ")
    _check_grad(_f64(dk), rk, "bwd split mqa dK")
    _check_grad(_f64(dv), rv, "bwd split mqa dV")


def test_split_deterministic_and_dq_unchanged():
    """Two split calls give the same bits; dQ (never split) equals fa2_bwd's bit for bit."""
    q, k, v = make_qkv(2, 8, 1000, 128, seed=530, H_kv=2)
    do = _dout(q.shape, 630)
    a = _grads(q, k, v, do, True, 0.088, True)
    b = _grads(q, k, v, do, True, 0.088, True)
    c = _grads(q, k, v, do, True, 0.088, False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(a[0], c[0])


def test_ws_entry_point_checks():
    """fa2_bwd_ws by symbol: the workspace rules of the header, then a valid call whose
    results equal the binding's."""
    lib = fa2.load_library()
    B, H, H_kv, N, d = 1, 8, 2, 512, 64
    q, k, v = make_qkv(B, H, N, d, seed=540, H_kv=H_kv)
    do = _dout(q.shape, 640)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa2.fwd_gqa(qd, kd, vd, causal=True)
    need = lib.fa2_bwd_workspace_bytes(B, H, H_kv, N, d, 1)
    assert need > 0
    ws = torch.empty(need + 16, dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    stream = int(torch.cuda.current_stream().cuda_stream)

    def call(ptr, nbytes):
        return lib.fa2_bwd_ws(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              dod.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                              B, H, H_kv, N, d, 1, float(1.0 / np.sqrt(d)), ptr, nbytes, stream)

    assert call(None, need) == 1                      # FA2_ERR_NULL_PTR
    assert call(ws.data_ptr() + 4, need) == 4         # FA2_ERR_MISALIGNED
    assert call(ws.data_ptr(), need - 1) == 10        # FA2_ERR_SCRATCH_TOO_SMALL
    assert call(ws.data_ptr(), need) == 0
    torch.cuda.synchronize()
    ref = fa2.bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_split_varlen(d):
    """fa2_bwd_varlen_ws: packed sequences (empty, one token, tile edges) over H=8 query heads
    and H_kv=2, plus 40 trailing tokens that no sequence covers: their dK/dV rows keep the
    value they had, the covered rows match the oracle and the unsplit call."""
    from oracle import attention_backward_varlen
    from synthetic import make_varlen
    H, H_kv, extra = 8, 2, 40
    q, k, v, cu, lengths = make_varlen(H, d, seed=550 + d, lengths=[1, 127, 0, 128, 129, 300, 64, 2], H_kv=H_kv)
    T0 = q.shape[1]
    pad = lambda t: torch.cat([t, torch.ones(t.shape[0], extra, d, dtype=t.dtype)], dim=1)
    q, k, v = pad(q), pad(k), pad(v)
    do = _dout(q.shape, 650 + d)
    scale = 1.0 / np.sqrt(d)
    lib = fa2.load_library()
    qd, kd, vd, dod, cud = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), cu.to(DEV)
    for causal in (False, True):
        need = lib.fa2_bwd_varlen_workspace_bytes(len(lengths), max(lengths), T0 + extra, H, H_kv, d, int(causal))
        assert need > 0, "shape does not exercise the split"
        tag = f"bwd split varlen d{d} causal={causal}"
        print(f"[case] {tag}", flush=True)
        o, lse = fa2.fwd_varlen_gqa(qd, kd, vd, cud, max(lengths), causal=causal, scale=scale)
        rq, rk, rv = attention_backward_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                               do.double().numpy(), cu.numpy(), causal, scale)
        outs = []
        for split in (True, False):
            dk = torch.full_like(kd, 7.0)
            dv = torch.full_like(vd, 7.0)
            dq, dk, dv = fa2.bwd_varlen(qd, kd, vd, o, lse, dod, cud, max(lengths), causal=causal, scale=scale,
                                        dk=dk, dv=dv, split=split)
            torch.cuda.synchronize()
            assert torch.all(dk[:, T0:] == 7.0) and torch.all(dv[:, T0:] == 7.0), tag + ": uncovered rows written"
            t = tag + (" ws" if split else " plain")
            _check_grad(_f64(dq[:, :T0]), rq[:, :T0], t + " dQ")
            _check_grad(_f64(dk[:, :T0]), rk[:, :T0], t + " dK")
            _check_grad(_f64(dv[:, :T0]), rv[:, :T0], t + " dV")
            outs.append((dq, dk, dv))
        assert torch.equal(outs[0][0][:, :T0], outs[1][0][:, :T0])     # dQ is never split (uncovered rows unset)
