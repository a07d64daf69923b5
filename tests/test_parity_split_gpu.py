"""GPU parity for key/value-chunk attention (fa2_fwd_chunk) and the LSE merge (fa2_lse_merge).

The chunk call is compared with oracle.attention_chunk (rows with no allowed key must come
back as O = 0 and LSE = -inf exactly); the merge kernel with oracle.lse_merge on the same
bf16/fp32 inputs; and split-KV end to end (chunks, then merge) with the oracle's full
attention and with the one-pass forward. Tolerances are the forward's (O max 2e-2, mean
2e-3; LSE 1e-3): a merged O carries the bf16 rounding of each part (half an ulp, <= 2^-8
relative) plus its own.
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention, attention_chunk, attention_rows, lse_merge
from synthetic import make_qkv

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
DEV = "cuda:0"


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o, l, o_ref, l_ref, tag):
    o, l = np.asarray(o, dtype=np.float64), np.asarray(l, dtype=np.float64)
    dead = ~np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(l), dead), f"{tag}: -inf rows differ"
    assert np.all(o[dead] == 0.0), f"{tag}: rows without keys must be zero"
    assert np.all(np.isfinite(o)), f"{tag}: non-finite O"
    err = np.abs(o - o_ref)
    lerr = np.abs(l[~dead] - l_ref[~dead])
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    lmx = float(lerr.max(initial=0.0))
    print(f"[parity] {tag}: O max {mx:.3e} mean {mean:.3e} | LSE max {lmx:.3e} | dead rows {int(dead.sum())}",
          flush=True)
    assert mx <= O_MAX and mean <= O_MEAN and lmx <= LSE_MAX, tag


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("nq,nk", [(1, 300), (100, 1), (257, 1000), (300, 0), (129, 129), (64, 200)])
def test_chunk_small(d, nq, nk):
    gen_q = make_qkv(1, 4, nq, d, seed=400 + nq + d)[0]
    _, k, v = make_qkv(1, 2, nk, d, seed=500 + nk + d)
    scale = 1.0 / np.sqrt(d)
    qn, kn, vn = gen_q.double().numpy(), k.double().numpy(), v.double().numpy()
    for causal in (False, True):
        # +-2^30: the documented extremes (every key allowed / none allowed)
        for diag in sorted({0, nk - nq, -50, 200, 1 << 30, -(1 << 30)}):
            o_ref, l_ref = attention_chunk(qn, kn, vn, causal, diag, scale)
            for variant in range(fa2.num_variants(d)):
                print(f"[case] chunk d={d} nq={nq} nk={nk} causal={causal} diag={diag} v{variant}", flush=True)
                o, l = fa2.fwd_chunk(gen_q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, diag=diag, scale=scale,
                                     variant=variant)
                torch.cuda.synchronize()
                _check(_f64(o), _f64(l), o_ref, l_ref, f"chunk d{d} {nq}x{nk} causal={causal} diag={diag} v{variant}")


@pytest.mark.parametrize("d", [40, 64, 96, 128, 192, 256])
def test_merge_kernel(d):
    """Both merge kernels: rows spread over lane groups (few parts or many rows) and one
    workgroup per row (4 or more parts over at most 4096 rows), on either side of the switch."""
    for S, rows in ((3, 1000), (5, 1000), (64, 37), (200, 5), (4, 4096), (8, 4097)):
        gen = torch.Generator(device="cpu").manual_seed(600 + d + S)
        o_parts = torch.randn((S, rows, d), generator=gen).to(torch.bfloat16)
        lse_parts = torch.randn((S, rows), generator=gen) * 4
        a, b = rows // 20, rows // 20 + max(rows // 100, 1)
        lse_parts[0, :a] = -float("inf")            # part 0 has no key for these rows
        lse_parts[:, a:b] = -float("inf")           # no part has a key for these rows
        lse_parts[1, b:b + max(rows // 100, 1)] += 80.0   # one part dominates
        o_parts[0, :a] = 0
        o_parts[:, a:b] = 0
        o_ref, l_ref = lse_merge(o_parts.double().numpy(), lse_parts.double().numpy())
        print(f"[case] merge d={d} parts={S} rows={rows}", flush=True)
        o, l = fa2.lse_merge(o_parts.to(DEV), lse_parts.to(DEV))
        torch.cuda.synchronize()
        _check(_f64(o), _f64(l), o_ref, l_ref, f"merge d{d} S{S} rows{rows}")


@pytest.mark.parametrize("causal", [False, True])
def test_split_kv_end_to_end(causal):
    B, H, N, d = 1, 8, 2048, 128
    q, k, v = make_qkv(B, H, N, d, seed=610)
    scale = 1.0 / np.sqrt(d)
    cuts = [0, 300, 1100, 1600, N]
    qd = q.to(DEV)
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = fa2.fwd_chunk(qd, k[:, :, a:b].contiguous().to(DEV), v[:, :, a:b].contiguous().to(DEV),
                             causal=causal, diag=-a, scale=scale)
        parts_o.append(o)
        parts_l.append(l)
    o, l = fa2.lse_merge(torch.stack(parts_o), torch.stack(parts_l))
    o_dir, l_dir = fa2.fwd(qd, k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    _check(_f64(o), _f64(l), o_ref, l_ref, f"split-kv 4 chunks causal={causal} vs oracle")
    _check(_f64(o), _f64(l), _f64(o_dir), _f64(l_dir), f"split-kv 4 chunks causal={causal} vs one pass")


def test_split_kv_long_and_decode():
    """Long-context causal shape (B=1 H=16 N=16384 d=128): 8 equal key chunks merged, against
    the one-pass forward (all rows) and the oracle (sampled rows); then the last 16 queries
    only (bottom-right alignment, diag = N_k - N_q), split the same way."""
    B, H, N, d = 1, 16, 16384, 128
    q, k, v = make_qkv(B, H, N, d, seed=4)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    step = N // 8
    for nq in (N, 16):
        qq = qd[:, :, N - nq:].contiguous()
        print(f"[case] split-kv long nq={nq}", flush=True)
        parts = [fa2.fwd_chunk(qq, kd[:, :, a:a + step].contiguous(), vd[:, :, a:a + step].contiguous(),
                               causal=True, diag=(N - nq) - a, scale=scale) for a in range(0, N, step)]
        o, l = fa2.lse_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
        o_dir, l_dir = fa2.fwd_chunk(qq, kd, vd, causal=True, diag=N - nq, scale=scale)
        torch.cuda.synchronize()
        _check(_f64(o), _f64(l), _f64(o_dir), _f64(l_dir), f"split-kv long nq={nq} vs one pass")
        rows = sorted({0, nq // 2, nq - 1, *np.random.default_rng(620).integers(0, nq, 6).tolist()})
        for h in (0, 9):
            o_ref, l_ref = attention_rows(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                          v[0, h].double().numpy(), True, scale, [N - nq + r for r in rows])
            _check(_f64(o[0, h, rows]), _f64(l[0, h, rows]), o_ref, l_ref, f"split-kv long nq={nq} h{h} vs oracle")


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("nq,nk", [(1, 1000), (16, 5000), (257, 1000), (100, 1), (130, 0)])
def test_splitkv_one_launch(d, nq, nk):
    q = make_qkv(1, 4, nq, d, seed=700 + nq + d)[0]
    _, k, v = make_qkv(1, 2, nk, d, seed=800 + nk + d)
    scale = 1.0 / np.sqrt(d)
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    variants = sorted({0, fa2.num_variants(d) - 1})        # default and ping-pong kernels
    for causal in (False, True):
        for diag in sorted({nk - nq, 0, -50}):
            o_ref, l_ref = attention_chunk(qn, kn, vn, causal, diag, scale)
            for splits in (1, 3, 8, 64):
                for variant in variants:
                    print(f"[case] splitkv d={d} nq={nq} nk={nk} causal={causal} diag={diag} S={splits} "
                          f"v{variant}", flush=True)
                    o, l = fa2.fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), splits, causal=causal, diag=diag,
                                           scale=scale, variant=variant)
                    torch.cuda.synchronize()
                    _check(_f64(o), _f64(l), o_ref, l_ref,
                           f"splitkv d{d} {nq}x{nk} causal={causal} diag={diag} S={splits} v{variant}")


def test_splitkv_long_decode():
    """Last 16 / 128 queries over the 16384 keys of the long-context shape, split 32 / 16 ways in
    one launch, against the one-pass chunk call (all rows) and the oracle (sampled rows)."""
    B, H, N, d = 1, 16, 16384, 128
    q, k, v = make_qkv(B, H, N, d, seed=4)
    scale = 1.0 / np.sqrt(d)
    kd, vd = k.to(DEV), v.to(DEV)
    for nq, S in ((16, 32), (128, 16)):
        qq = q[:, :, N - nq:].contiguous().to(DEV)
        print(f"[case] splitkv long nq={nq} S={S}", flush=True)
        o, l = fa2.fwd_splitkv(qq, kd, vd, S, causal=True, diag=N - nq, scale=scale)
        o_dir, l_dir = fa2.fwd_chunk(qq, kd, vd, causal=True, diag=N - nq, scale=scale)
        torch.cuda.synchronize()
        _check(_f64(o), _f64(l), _f64(o_dir), _f64(l_dir), f"splitkv long nq={nq} S={S} vs one pass")
        rows = [0, nq // 2, nq - 1]
        for h in (3, 14):
            o_ref, l_ref = attention_rows(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                          v[0, h].double().numpy(), True, scale, [N - nq + r for r in rows])
            _check(_f64(o[0, h, rows]), _f64(l[0, h, rows]), o_ref, l_ref, f"splitkv long nq={nq} h{h} vs oracle")


def test_merge_rejects_bad_arguments():
    o = torch.zeros((2, 10, 100), dtype=torch.bfloat16, device=DEV)
    l = torch.zeros((2, 10), device=DEV)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.lse_merge(o, l)
    assert e.value.status == 3
