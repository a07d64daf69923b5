"""GPU parity for grouped-query and multi-query attention (fa2_fwd_gqa, fa2_fwd_varlen_gqa).

Query head h reads key/value head floor(h / g), g = H / H_kv (chlience notes §5.6). The
oracle is oracle.attention_gqa / attention_varlen_gqa (fp64); tolerances are those of
test_parity_gpu.py. A second, size-independent check: the kernel's GQA result must equal,
bit for bit, its own multi-head result on K/V whose heads were copied out explicitly (the
same arithmetic on the same values in the same order).
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_gqa, attention_rows, attention_varlen_gqa, kv_head
from synthetic import make_qkv, make_varlen

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
DEV = "cuda:0"


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o_gpu, l_gpu, o_ref, l_ref, tag):
    o, l = np.asarray(o_gpu, dtype=np.float64), np.asarray(l_gpu, dtype=np.float64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{tag}: non-finite output"
    err, lerr = np.abs(o - o_ref), np.abs(l - l_ref)
    mx, mean, lmx = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0, float(lerr.max(initial=0.0))
    print(f"[parity] {tag}: O max {mx:.3e} mean {mean:.3e} | LSE max {lmx:.3e}", flush=True)
    assert mx <= O_MAX and mean <= O_MEAN and lmx <= LSE_MAX, tag


@pytest.mark.parametrize("d", [64, 80, 128, 256])
@pytest.mark.parametrize("H,H_kv", [(8, 1), (8, 2), (6, 3), (8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_small(d, H, H_kv, causal):
    N = 257   # three 128-row blocks, the last one ragged
    q, k, v = make_qkv(2, H, N, d, seed=100 + H * 10 + H_kv, H_kv=H_kv)
    scale = 1.0 / np.sqrt(d)
    o_ref, l_ref = attention_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    for variant in range(fa2.num_variants(d)):
        print(f"[case] gqa d={d} H={H} H_kv={H_kv} causal={causal} variant={variant}", flush=True)
        o, l = fa2.fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, variant=variant)
        torch.cuda.synchronize()
        _check(_f64(o), _f64(l), o_ref, l_ref, f"gqa d{d} H{H}/{H_kv} causal={causal} v{variant}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_gqa_varlen(d):
    lengths = [1, 127, 0, 128, 129, 300, 64, 2]
    H, H_kv = 8, 2
    q, k, v, cu, lengths = make_varlen(H, d, seed=140 + d, lengths=lengths, H_kv=H_kv)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        o_ref, l_ref = attention_varlen_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                            cu.numpy(), causal, scale)
        for variant in range(fa2.num_variants(d)):
            print(f"[case] gqa varlen d={d} causal={causal} variant={variant}", flush=True)
            o, l = fa2.fwd_varlen_gqa(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths),
                                      causal=causal, scale=scale, variant=variant)
            torch.cuda.synchronize()
            _check(_f64(o), _f64(l), o_ref, l_ref, f"gqa varlen d{d} causal={causal} v{variant}")


def test_gqa_equals_mha_on_copied_heads():
    """Bitwise: GQA on [B, H_kv] K/V == MHA on the same K/V heads copied out to [B, H]."""
    B, H, H_kv, N, d = 2, 16, 4, 1000, 128
    q, k, v = make_qkv(B, H, N, d, seed=150, H_kv=H_kv)
    idx = torch.tensor([kv_head(h, H, H_kv) for h in range(H)])
    k_full, v_full = k[:, idx].contiguous(), v[:, idx].contiguous()
    for causal in (False, True):
        print(f"[case] gqa==mha causal={causal}", flush=True)
        o1, l1 = fa2.fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        o2, l2 = fa2.fwd(q.to(DEV), k_full.to(DEV), v_full.to(DEV), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_long_sampled():
    """B=1, 32 query heads over 8 K/V heads, N=8192, d=128, causal: sampled rows."""
    B, H, H_kv, N, d = 1, 32, 8, 8192, 128
    q, k, v = make_qkv(B, H, N, d, seed=160, H_kv=H_kv)
    scale = 1.0 / np.sqrt(d)
    print("[case] gqa long B1 H32/8 N8192 d128 causal", flush=True)
    o, l = fa2.fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    o, l = _f64(o), _f64(l)
    rng = np.random.default_rng(161)
    rows = sorted({0, 1, 127, 128, 4095, 4096, N - 1, *rng.integers(0, N, 12).tolist()})
    for h in (0, 3, 4, 17, 31):
        hk = kv_head(h, H, H_kv)
        o_ref, l_ref = attention_rows(q[0, h].double().numpy(), k[0, hk].double().numpy(),
                                      v[0, hk].double().numpy(), True, scale, rows)
        _check(o[0, h, rows], l[0, h, rows], o_ref, l_ref, f"gqa long h{h}->kv{hk}")


def test_gqa_rejects_bad_groups():
    q, k, v = make_qkv(1, 6, 64, 64, seed=170, H_kv=4)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV))
    assert e.value.status == 2
