"""GPU parity: the gfx950 kernels (through the C ABI) against the CPU fp64 oracle.

Tolerances (fixed by the task's benchmark spec, not derived here):
  O:   max |O_gpu - O_ref| <= 2e-2 and mean |O_gpu - O_ref| <= 2e-3 over all compared elements
  LSE: max |LSE_gpu - LSE_ref| <= 1e-3
The GPU O is bf16, so its own rounding (<= half an ulp, 2^-8 relative) is inside these.

Coverage: the five benchmark workloads (the single-head one fully; the others at full size on sampled rows that
the oracle computes one by one, including row-block edges and the last rows), odd and ragged
shapes spanning several tiles, every kernel variant, packed variable-length batches with
empty/1-token/tile-edge sequences, scale edge cases, large score ranges, row maxima that
move on every key tile (or never), long sequences, determinism and batch invariance.
"""
import math

import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention, attention_rows, attention_varlen
from synthetic import WORKLOADS, make_qkv, make_varlen, workload_inputs

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
DEV = "cuda:0"


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o_gpu, l_gpu, o_ref, l_ref, tag):
    o, l = np.asarray(o_gpu, dtype=np.float64), np.asarray(l_gpu, dtype=np.float64)
    assert np.all(np.isfinite(o)), f"{tag}: non-finite O"
    assert np.all(np.isfinite(l)), f"{tag}: non-finite LSE"
    err = np.abs(o - o_ref)
    lerr = np.abs(l - l_ref)
    mx, mean, lmx = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0, float(lerr.max(initial=0.0))
    print(f"[parity] {tag}: O max {mx:.3e} mean {mean:.3e} | LSE max {lmx:.3e}", flush=True)
    assert mx <= O_MAX, f"{tag}: O max-abs {mx}"
    assert mean <= O_MEAN, f"{tag}: O mean-abs {mean}"
    assert lmx <= LSE_MAX, f"{tag}: LSE max-abs {lmx}"


def _run_fixed(q, k, v, causal, scale, variant=0):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = fa2.fwd(qd, kd, vd, causal=causal, scale=scale, variant=variant)
    torch.cuda.synchronize()
    return o, l


def _sample_rows(N, rng, extra=24):
    base = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 65, N - 64,
            N - 2, N - 1]
    base += list(rng.integers(0, N, size=extra))
    return sorted({int(r) for r in base if 0 <= r < N})


def test_single_head_full():
    w = WORKLOADS["single_head_256"]
    q, k, v = workload_inputs(w)
    o, l = _run_fixed(q, k, v, w.causal, w.scale)
    o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.causal, w.scale)
    _check(_f64(o), _f64(l), o_ref, l_ref, "single_head_256 full")


@pytest.mark.parametrize("name", ["batch8_2k_d128", "batch8_2k_d64_causal", "long_16k_causal"])
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    print(f"[parity] {name}: {w.description}", flush=True)
    q, k, v = workload_inputs(w)
    o, l = _run_fixed(q, k, v, w.causal, w.scale)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(l).all())
    rng = np.random.default_rng(100 + w.seed)
    pairs = sorted({(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))})
    for b, h in pairs:
        rows = _sample_rows(w.N, rng)
        o_ref, l_ref = attention_rows(q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                                      w.causal, w.scale, rows)
        _check(_f64(o[b, h, rows]), _f64(l[b, h, rows]), o_ref, l_ref, f"{name} b{b} h{h} {len(rows)} rows")


@pytest.mark.parametrize("name", ["batch8_2k_d128", "batch8_2k_d64_causal", "long_16k_causal"])
def test_full_size_every_variant_sampled(name):
    """Every kernel variant at the benchmark sizes, on rows sampled from one (batch, head)
    pair (the first, the last row-block edges and random rows)."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rng = np.random.default_rng(200 + w.seed)
    b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
    rows = _sample_rows(w.N, rng, extra=8)
    o_ref, l_ref = attention_rows(q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                                  w.causal, w.scale, rows)
    for variant in range(fa2.num_variants(w.d)):
        print(f"[case] {name} v{variant} ({fa2.variant_name(w.d, variant)})", flush=True)
        o, l = fa2.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, variant=variant)
        torch.cuda.synchronize()
        _check(_f64(o[b, h, rows]), _f64(l[b, h, rows]), o_ref, l_ref, f"{name} v{variant} b{b} h{h}")


def test_varlen16_every_variant_sampled():
    w = WORKLOADS["varlen16_causal"]
    q, k, v, cu, lengths = workload_inputs(w)
    qd, kd, vd, cud = q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV)
    rng = np.random.default_rng(106)
    s = int(np.argmax(lengths))
    a, e = int(cu[s]), int(cu[s + 1])
    h = int(rng.integers(w.H))
    rows = _sample_rows(e - a, rng, extra=8)
    o_ref, l_ref = attention_rows(q[h, a:e].double().numpy(), k[h, a:e].double().numpy(), v[h, a:e].double().numpy(),
                                  True, w.scale, rows)
    idx = [a + r for r in rows]
    for variant in range(fa2.num_variants(w.d)):
        print(f"[case] varlen16 v{variant}", flush=True)
        o, l = fa2.fwd_varlen(qd, kd, vd, cud, max(lengths), causal=True, scale=w.scale, variant=variant)
        torch.cuda.synchronize()
        _check(_f64(o[h, idx]), _f64(l[h, idx]), o_ref, l_ref, f"varlen16 v{variant} seq{s} h{h}")


def test_varlen16_sampled():
    w = WORKLOADS["varlen16_causal"]
    q, k, v, cu, lengths = workload_inputs(w)
    print(f"[parity] varlen16_causal lengths {lengths} T={sum(lengths)}", flush=True)
    o, l = fa2.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(l).all())
    rng = np.random.default_rng(105)
    seqs = sorted({int(np.argmax(lengths)), int(np.argmin(lengths)), int(rng.integers(len(lengths))), 0,
                   len(lengths) - 1})
    for s in seqs:
        a, b = int(cu[s]), int(cu[s + 1])
        for h in (0, w.H - 1):
            rows = _sample_rows(b - a, rng, extra=16)
            o_ref, l_ref = attention_rows(q[h, a:b].double().numpy(), k[h, a:b].double().numpy(),
                                          v[h, a:b].double().numpy(), True, w.scale, rows)
            idx = [a + r for r in rows]
            _check(_f64(o[h, idx]), _f64(l[h, idx]), o_ref, l_ref, f"varlen seq{s} len{b - a} h{h}")


ODD_N = [1, 17, 100, 128, 129, 255, 1000]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", ODD_N)
def test_odd_shapes_full(N, d, causal):
    q, k, v = make_qkv(2, 3, N, d, seed=1000 + N + d + int(causal))
    scale = 1.0 / math.sqrt(d)
    for variant in range(fa2.num_variants(d)):
        o, l = _run_fixed(q, k, v, causal, scale, variant)
        o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
        _check(_f64(o), _f64(l), o_ref, l_ref, f"N{N} d{d} causal{int(causal)} {fa2.variant_name(d, variant)}")


@pytest.mark.parametrize("d", [8, 32, 80, 96, 160, 192, 248])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_not_64_128_256(d, causal):
    """Head dims that are multiples of 8 run on the next kernel width with padded columns."""
    for N in (1, 129, 300):
        q, k, v = make_qkv(2, 3, N, d, seed=2000 + N + d + int(causal))
        scale = 1.0 / math.sqrt(d)
        o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
        for variant in range(fa2.num_variants(d)):
            o, l = _run_fixed(q, k, v, causal, scale, variant)
            _check(_f64(o), _f64(l), o_ref, l_ref, f"N{N} d{d} causal{int(causal)} {fa2.variant_name(d, variant)}")


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_edges_full(d, causal):
    lengths = [1, 127, 0, 128, 129, 5, 300, 64, 255, 256, 1000, 2]
    q, k, v, cu, lengths = make_varlen(2, d, seed=77 + d, lengths=lengths)
    scale = 1.0 / math.sqrt(d)
    for variant in range(fa2.num_variants(d)):
        o, l = fa2.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths) + 37, causal=causal,
                              scale=scale, variant=variant)
        torch.cuda.synchronize()
        o_ref, l_ref = attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(), cu.numpy(),
                                        causal, scale)
        _check(_f64(o), _f64(l), o_ref, l_ref, f"varlen d{d} causal{int(causal)} {fa2.variant_name(d, variant)}")


def test_varlen_k_scaled_by_3():
    q, k, v, cu, lengths = make_varlen(4, 128, seed=5, lengths=[700, 129, 1500, 64], k_scale=3.0)
    o, l = fa2.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths), causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(), cu.numpy(), True,
                                    1.0 / math.sqrt(128))
    _check(_f64(o), _f64(l), o_ref, l_ref, "varlen K x3")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_scale_edges(scale):
    q, k, v = make_qkv(1, 2, 200, 64, seed=31)
    for causal in (False, True):
        o, l = _run_fixed(q, k, v, causal, scale)
        o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                 float(np.float32(scale)))
        _check(_f64(o), _f64(l), o_ref, l_ref, f"scale {scale} causal{int(causal)}")


def test_large_scores():
    q, k, v = make_qkv(1, 2, 333, 128, seed=32)
    q, k = (q.float() * 4).to(torch.bfloat16), (k.float() * 4).to(torch.bfloat16)
    for causal in (False, True):
        o, l = _run_fixed(q, k, v, causal, 1 / math.sqrt(128))
        o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                 1 / math.sqrt(128))
        _check(_f64(o), _f64(l), o_ref, l_ref, f"scores x16 causal{int(causal)}")


@pytest.mark.parametrize("pattern", ["rising", "falling", "zigzag"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_moving_row_max(d, pattern):
    """Scores built so that the row maximum moves by 10 (in log2 units) with every 64 keys
    (rising), never moves after the first keys (falling: later tiles underflow), or rises on
    every other tile (zigzag). The reference max of the optimistic and lazy bookkeeping is
    then moved and the accumulator rescaled on every tile, or never. All variants against
    the oracle."""
    N, scale = 700, 1.0 / math.sqrt(d)
    c = scale * math.log2(math.e)
    j = torch.arange(N, dtype=torch.float64)
    t = j * (10.0 / (64.0 * c))                       # q.k grows by 10/c per 64 keys
    if pattern == "falling":
        t = -t
    elif pattern == "zigzag":
        t = torch.where((j // 64) % 2 == 0, t, -t)
    gen = torch.Generator().manual_seed(41 + d)
    q = (1.0 + 0.05 * torch.randn((1, 2, N, d), generator=gen)).to(torch.bfloat16)
    k = ((t / d)[None, None, :, None] + 0.01 * torch.randn((1, 2, N, d), generator=gen, dtype=torch.float64))
    k = k.float().to(torch.bfloat16)
    v = torch.randn((1, 2, N, d), generator=gen).to(torch.bfloat16)
    for causal in (False, True):
        o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
        for variant in range(fa2.num_variants(d)):
            print(f"[case] moving max {pattern} d={d} causal={causal} v{variant}", flush=True)
            o, l = _run_fixed(q, k, v, causal, scale, variant)
            _check(_f64(o), _f64(l), o_ref, l_ref, f"{pattern} d{d} causal{int(causal)} v{variant}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_long_sequence_sampled(d):
    N = 65537
    q, k, v = make_qkv(1, 2, N, d, seed=33)
    rng = np.random.default_rng(34)
    for causal in (True, False):
        o, l = _run_fixed(q, k, v, causal, 1 / math.sqrt(d))
        rows = _sample_rows(N, rng, extra=8)
        for h in (0, 1):
            o_ref, l_ref = attention_rows(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                          v[0, h].double().numpy(), causal, 1 / math.sqrt(d), rows)
            _check(_f64(o[0, h, rows]), _f64(l[0, h, rows]), o_ref, l_ref, f"N{N} d{d} causal{int(causal)} h{h}")


@pytest.mark.parametrize("d", [64, 128])
def test_million_token_sampled(d):
    """One causal head of 2^20 tokens: 16384 key tiles per row block and fp32 running sums
    over up to 2^20 keys. Sampled rows (first and last rows, tile edges, random rows) against
    the oracle, computed row by row."""
    N = 1 << 20
    q, k, v = make_qkv(1, 1, N, d, seed=36)
    scale = 1 / math.sqrt(d)
    print(f"[case] million-token causal d={d}", flush=True)
    o, l = _run_fixed(q, k, v, True, scale)
    rows = _sample_rows(N, np.random.default_rng(37), extra=6)
    o_ref, l_ref = attention_rows(q[0, 0].double().numpy(), k[0, 0].double().numpy(), v[0, 0].double().numpy(),
                                  True, scale, rows)
    _check(_f64(o[0, 0, rows]), _f64(l[0, 0, rows]), o_ref, l_ref, f"N{N} d{d} causal")


def test_deterministic_and_batch_invariant():
    q, k, v = make_qkv(3, 5, 300, 128, seed=35)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o1, l1 = fa2.fwd(qd, kd, vd, causal=causal)
        o2, l2 = fa2.fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "repeat run differs"
        o3, l3 = fa2.fwd(qd[1:2, 2:3].contiguous(), kd[1:2, 2:3].contiguous(), vd[1:2, 2:3].contiguous(),
                         causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1[1:2, 2:3], o3) and torch.equal(l1[1:2, 2:3], l3), "result depends on B/H"


def test_empty_and_preallocated():
    q = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, l = fa2.fwd(q, q, q, causal=True)
    assert o.shape == (2, 3, 0, 64) and l.shape == (2, 3, 0)
    qv = torch.zeros(2, 0, 128, dtype=torch.bfloat16, device=DEV)
    o, l = fa2.fwd_varlen(qv, qv, qv, torch.zeros(1, dtype=torch.int32, device=DEV), 0)
    assert o.shape == (2, 0, 128)
    q, k, v = make_qkv(1, 1, 64, 64, seed=36)
    out = torch.full((1, 1, 64, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, 1, 64), float("nan"), dtype=torch.float32, device=DEV)
    o, l = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), out=out, lse=lse)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_equal_lengths_equals_fixed_batch(d):
    """A fixed [B, H, N, d] batch and the same data packed as B varlen sequences of N tokens
    run under different grid orders (per-XCD pair ranges vs plain heaviest-first) and must
    agree bit for bit: every row's arithmetic is independent of where its workgroup runs."""
    B, H, N = 4, 8, 300
    q, k, v = make_qkv(B, H, N, d, seed=37)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous().to(DEV)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    for causal in (False, True):
        o, l = fa2.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        ov, lv = fa2.fwd_varlen(pack(q), pack(k), pack(v), cu, N, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, ov.reshape(H, B, N, d).permute(1, 0, 2, 3)), f"O d{d} causal={causal}"
        assert torch.equal(l, lv.reshape(H, B, N).permute(1, 0, 2)), f"LSE d{d} causal={causal}"
