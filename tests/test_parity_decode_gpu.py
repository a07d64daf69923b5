"""GPU parity for split-KV calls with few query rows per key/value head (decoding shapes).

One to four query rows per key/value head (query heads of a group times query rows) against
key sequences from 1 to 16384 keys, cut into 2 to 64 pieces that run in one launch and are
merged by LSE (the per-row merge kernel takes over from 4 pieces). Every case is compared over
all elements with oracle.attention_chunk (the materialised definition with the chunk's causal
offset; rows with no allowed key must be O = 0, LSE = -inf exactly), and the default variant
with the 4-wave tiled variant (variant 1) on the same inputs. Tolerances are the forward's:
O max 2e-2 and mean 2e-3, LSE max 1e-3.
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_chunk
from synthetic import make_qkv

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
DEV = "cuda:0"


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o, l, o_ref, l_ref, tag):
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


def _run(B, H, H_kv, nq, nk, d, causal, diag, splits, scale, seed, k_scale=1.0):
    q = make_qkv(B, H, nq, d, seed=seed)[0]
    _, k, v = make_qkv(B, H_kv, nk, d, seed=seed + 1)
    if k_scale != 1.0:
        k = (k.float() * k_scale).to(torch.bfloat16)
    o_ref, l_ref = attention_chunk(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, diag, scale)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    tag = f"decode B{B} H{H}/{H_kv} nq={nq} nk={nk} d={d} causal={causal} diag={diag} S={splits} scale={scale:.3g}"
    print(f"[case] {tag}", flush=True)
    o, l = fa2.fwd_splitkv(qd, kd, vd, splits, causal=causal, diag=diag, scale=scale)
    o_t, l_t = fa2.fwd_splitkv(qd, kd, vd, splits, causal=causal, diag=diag, scale=scale, variant=1)
    torch.cuda.synchronize()
    _check(_f64(o), _f64(l), o_ref, l_ref, tag)
    _check(_f64(o), _f64(l), _f64(o_t), _f64(l_t), tag + " vs tiled")


@pytest.mark.parametrize("d", [8, 64, 96, 128, 200, 256])
@pytest.mark.parametrize("H,H_kv,nq", [(4, 4, 1), (8, 2, 1), (6, 3, 2), (4, 4, 3), (8, 8, 4), (4, 1, 1)])
def test_decode_shapes(d, H, H_kv, nq):
    for nk in (1, 37, 1000, 4097):
        for causal in (False, True):
            for splits in (2, 7, 64):
                _run(2, H, H_kv, nq, nk, d, causal, nk - nq, splits, 1.0 / np.sqrt(d), seed=11 * d + nk + nq)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_offsets_and_scales(d):
    """Causal offsets that leave rows without keys in some or all pieces, negative and zero
    scale, and scores stretched by K x 3."""
    for diag in (-3, 0, 5, 1 << 30, -(1 << 30)):
        _run(1, 4, 2, 2, 300, d, True, diag, 5, 1.0 / np.sqrt(d), seed=3 + d)
    for scale in (-0.3, 0.0, 0.9):
        _run(1, 4, 4, 1, 500, d, False, 0, 8, scale, seed=5 + d)
    _run(1, 8, 2, 1, 3000, d, True, 2999, 16, 1.0 / np.sqrt(d), seed=7 + d, k_scale=3.0)


def test_decode_long_context():
    """One new token against the 16384 keys of the long-context shape (B=1, H=16, d=128),
    bottom-right causal, 64 pieces: every row against the oracle."""
    B, H, N, d = 1, 16, 16384, 128
    q, k, v = make_qkv(B, H, N, d, seed=4)
    qq = q[:, :, N - 1:].contiguous()
    scale = 1.0 / np.sqrt(d)
    o_ref, l_ref = attention_chunk(qq.double().numpy(), k.double().numpy(), v.double().numpy(), True, N - 1, scale)
    print("[case] decode long context", flush=True)
    o, l = fa2.fwd_splitkv(qq.to(DEV), k.to(DEV), v.to(DEV), 64, causal=True, diag=N - 1, scale=scale)
    torch.cuda.synchronize()
    _check(_f64(o), _f64(l), o_ref, l_ref, "decode long context")


def test_decode_noalloc_matches_workspace_call():
    """The no-allocation entry point gives the workspace call's results bit for bit."""
    q = make_qkv(2, 8, 1, 128, seed=21)[0]
    _, k, v = make_qkv(2, 2, 5000, 128, seed=22)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    print("[case] decode no-alloc", flush=True)
    o, l = fa2.fwd_splitkv(qd, kd, vd, 32, causal=True, diag=4999)
    o2, l2 = torch.empty_like(o), torch.empty_like(l)
    lib = fa2.load_library()
    st = lib.fa2_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                     2, 8, 2, 1, 5000, 128, 1, 4999, float(1.0 / np.sqrt(128)), 32, 0,
                                     int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, lib.fa2_status_str(st).decode()
    assert torch.equal(o, o2) and torch.equal(l, l2)
