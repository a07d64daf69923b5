"""GPU parity for the backward (fa2_bwd, fa2_bwd_varlen) against the CPU fp64 oracle.

Inputs Q, K, V, dO are seeded bf16; O and LSE come from the GPU forward (as in training);
the oracle (oracle.attention_backward_gqa / _varlen) differentiates the exact definition in
fp64 from Q, K, V, dO alone.

Tolerance. No tolerance is stated for gradients, so one is derived from the arithmetic:
the kernels feed P and dS to the matrix cores as bf16 (relative rounding <= 2^-8 per
entry, the unit roundoff of an 8-bit significand), accumulate in fp32 and round the
gradients to bf16 (another 2^-8); D is formed from the forward's bf16 O (relative error
<= 2^-8 per element). Each gradient entry is a sum of many such terms of mixed sign, so its
error is a few 2^-8 of the magnitude of the terms, not of the (possibly cancelled) sum. The test therefore bounds the error relative to the
largest reference entry of the tensor:
    max |g - g_ref| <= 2e-2 * max |g_ref|      (~5 x 2^-8)
    mean|g - g_ref| <= 2e-3 * max |g_ref|
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_backward_gqa, attention_backward_head, attention_backward_varlen
from synthetic import make_qkv, make_varlen

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
    mx = float(err.max(initial=0.0))
    mean = float(err.mean()) if err.size else 0.0
    rel_mx = mx / scale if scale > 0 else mx
    rel_mean = mean / scale if scale > 0 else mean
    print(f"[parity] {tag}: max {mx:.3e} ({rel_mx:.2e} of max|ref| {scale:.3e}) mean {rel_mean:.2e}", flush=True)
    assert rel_mx <= G_MAX, f"{tag}: max error {rel_mx:.3e} of max|ref|"
    assert rel_mean <= G_MEAN, f"{tag}: mean error {rel_mean:.3e} of max|ref|"


def _run(q, k, v, do, causal, scale):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    if k.shape[1] == q.shape[1]:
        o, lse = fa2.fwd(qd, kd, vd, causal=causal, scale=scale)
    else:
        o, lse = fa2.fwd_gqa(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa2.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _compare(q, k, v, do, causal, scale, tag):
    dq, dk, dv = _run(q, k, v, do, causal, scale)
    rq, rk, rv = attention_backward_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        do.double().numpy(), causal, scale)
    _check_grad(_f64(dq), rq, tag + " dQ")
    _check_grad(_f64(dk), rk, tag + " dK")
    _check_grad(_f64(dv), rv, tag + " dV")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 17, 100, 128, 129, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small(d, N, causal):
    q, k, v = make_qkv(2, 4, N, d, seed=200 + N + d)
    do = _dout(q.shape, 300 + N + d)
    print(f"[case] bwd d={d} N={N} causal={causal}", flush=True)
    _compare(q, k, v, do, causal, 1.0 / np.sqrt(d), f"bwd d{d} N{N} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("H_kv", [1, 2])
def test_bwd_gqa(d, H_kv):
    q, k, v = make_qkv(2, 4, 300, d, seed=210 + H_kv + d, H_kv=H_kv)
    do = _dout(q.shape, 310 + H_kv + d)
    for causal in (False, True):
        print(f"[case] bwd gqa d={d} H_kv={H_kv} causal={causal}", flush=True)
        _compare(q, k, v, do, causal, 1.0 / np.sqrt(d), f"bwd gqa d{d} 4/{H_kv} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bwd_varlen(d):
    lengths = [1, 127, 0, 128, 129, 300, 64, 2]
    H, H_kv = 4, 2
    q, k, v, cu, lengths = make_varlen(H, d, seed=220 + d, lengths=lengths, H_kv=H_kv)
    do = _dout(q.shape, 320 + d)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        print(f"[case] bwd varlen d={d} causal={causal}", flush=True)
        qd, kd, vd, dod, cud = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), cu.to(DEV)
        o, lse = fa2.fwd_varlen_gqa(qd, kd, vd, cud, max(lengths), causal=causal, scale=scale)
        dq, dk, dv = fa2.bwd_varlen(qd, kd, vd, o, lse, dod, cud, max(lengths), causal=causal, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv = attention_backward_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                               do.double().numpy(), cu.numpy(), causal, scale)
        tag = f"bwd varlen d{d} causal={causal}"
        _check_grad(_f64(dq), rq, tag + " dQ")
        _check_grad(_f64(dk), rk, tag + " dK")
        _check_grad(_f64(dv), rv, tag + " dV")


@pytest.mark.parametrize("d", [8, 32, 80, 96, 136, 200, 248])
def test_bwd_padded_head_dims(d):
    """Head dims that are multiples of 8 below 256 run on the 64/128/256 kernels with padding."""
    for N, H_kv in ((100, 4), (257, 2)):
        q, k, v = make_qkv(2, 4, N, d, seed=260 + N + d, H_kv=H_kv)
        do = _dout(q.shape, 360 + N + d)
        for causal in (False, True):
            print(f"[case] bwd padded d={d} N={N} H_kv={H_kv} causal={causal}", flush=True)
            _compare(q, k, v, do, causal, 1.0 / np.sqrt(d), f"bwd d{d} N{N} 4/{H_kv} causal={causal}")


def test_bwd_scale_edges():
    q, k, v = make_qkv(1, 2, 200, 64, seed=230)
    do = _dout(q.shape, 330)
    for scale in (-0.09, 0.0, 0.5):
        for causal in (False, True):
            print(f"[case] bwd scale={scale} causal={causal}", flush=True)
            _compare(q, k, v, do, causal, scale, f"bwd scale={scale} causal={causal}")


def test_bwd_long_full_heads():
    """The long-context causal shape (B=1 H=16 N=16384 d=128) in one launch; head 11
    compared in full against the oracle."""
    B, H, N, d = 1, 16, 16384, 128
    q, k, v = make_qkv(B, H, N, d, seed=4)
    do = _dout(q.shape, 340)
    scale = 1.0 / np.sqrt(d)
    print("[case] bwd long B1 H16 N16384 d128 causal", flush=True)
    dq, dk, dv = _run(q, k, v, do, True, scale)
    for h in (11,):
        rq, rk, rv = attention_backward_head(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                             v[0, h].double().numpy(), do[0, h].double().numpy(), True, scale)
        _check_grad(_f64(dq[0, h]), rq, f"bwd long h{h} dQ")
        _check_grad(_f64(dk[0, h]), rk, f"bwd long h{h} dK")
        _check_grad(_f64(dv[0, h]), rv, f"bwd long h{h} dV")
        del rq, rk, rv


def test_bwd_d256_long_full_head():
    """d = 256 (one wave per SIMD in both kernels) over 4096 causal rows, four heads in one
    launch; head 2 compared in full against the oracle."""
    B, H, N, d = 1, 4, 4096, 256
    q, k, v = make_qkv(B, H, N, d, seed=270)
    do = _dout(q.shape, 370)
    scale = 1.0 / np.sqrt(d)
    print("[case] bwd B1 H4 N4096 d256 causal", flush=True)
    dq, dk, dv = _run(q, k, v, do, True, scale)
    h = 2
    rq, rk, rv = attention_backward_head(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                         v[0, h].double().numpy(), do[0, h].double().numpy(), True, scale)
    _check_grad(_f64(dq[0, h]), rq, "bwd d256 long dQ")
    _check_grad(_f64(dk[0, h]), rk, "bwd d256 long dK")
    _check_grad(_f64(dv[0, h]), rv, "bwd d256 long dV")


def test_bwd_deterministic():
    q, k, v = make_qkv(2, 8, 1000, 128, seed=240, H_kv=2)
    do = _dout(q.shape, 340)
    a = _run(q, k, v, do, True, 0.088)
    b = _run(q, k, v, do, True, 0.088)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_rejects_bad_shapes():
    q, k, v = make_qkv(1, 6, 64, 64, seed=250, H_kv=4)
    qd = q.to(DEV)
    lse = torch.zeros(1, 6, 64, device=DEV)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.bwd(qd, k.to(DEV), v.to(DEV), qd, lse, qd)
    assert e.value.status == 2


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_varlen_equal_lengths_equals_fixed_batch(d):
    """The fixed-length and varlen backward (different grid orders) agree bit for bit on a
    batch packed as equal-length sequences."""
    B, H, N = 4, 8, 300
    q, k, v = make_qkv(B, H, N, d, seed=280)
    do = _dout(q.shape, 380)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous().to(DEV)
    unpack = lambda t: t.reshape(H, B, N, d).permute(1, 0, 2, 3)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    for causal in (False, True):
        dq, dk, dv = _run(q, k, v, do, causal, 1.0 / np.sqrt(d))
        o, lse = fa2.fwd_varlen(pack(q), pack(k), pack(v), cu, N, causal=causal)
        gv = fa2.bwd_varlen(pack(q), pack(k), pack(v), o, lse, pack(do), cu, N, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), gv):
            assert torch.equal(a, unpack(b)), f"{name} d{d} causal={causal}"
