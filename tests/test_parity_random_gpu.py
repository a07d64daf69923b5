"""Randomised GPU parity sweep against the fp64 oracle.

Shapes and options are drawn from one seeded generator: B, H, H_kv (a divisor of H), a
ragged N, any head dimension that is a multiple of 8 up to 256, a scale of either sign,
causal or not, the kernel variant, and packed variable-length batches with empty,
one-token and tile-edge sequences. Every case runs on the GPU and in the oracle on the
same inputs. One case in three also runs the backward. The forward is held to the stated
tolerances (O max 2e-2, mean 2e-3; LSE 1e-3); the backward to the backward parity
tests' bound, relative to the largest reference entry (max 2e-2, mean 2e-3). The cases
are small enough for the oracle to finish in seconds; larger shapes are covered by the
fixed parity tests.

The largest O errors come from draws with a large scale and head dimension (score spread
about 6), where a row's softmax is dominated by one key and O is close to that key's V row.
The kernel divides O by the sum of the bf16 weights the PV product actually consumed, so the
rounding of the dominant weight cancels; what remains is O's own bf16 rounding (half an ulp,
up to 2^-8 relative: 1.6e-2 for |O| just under 8, 7.8e-3 under 4) and the rounding of the
small weights. Before that normalisation the bf16 dominant weight against an fp32 row sum
added up to 2^-8 * |V| more, and this sweep's worst draw measured 1.85e-2; now 1.39e-2.
"""

import numpy as np
import pytest
import torch

import exact_softmax_attention_amd as fa2
from oracle import attention_backward_gqa, attention_gqa, attention_varlen_gqa
from synthetic import make_qkv, make_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
G_MAX, G_MEAN = 2e-2, 2e-3
CASES = 48


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check_fwd(o, l, o_ref, l_ref, tag):
    o, l = _f64(o), _f64(l)
    live = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), live), f"{tag}: -inf rows differ"
    err = np.abs(o - o_ref)
    lerr = np.abs(l[live] - l_ref[live])
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    lmx = float(lerr.max(initial=0.0))
    print(f"[parity] {tag}: O max {mx:.2e} mean {mean:.2e} LSE {lmx:.2e}", flush=True)
    assert mx <= O_MAX and mean <= O_MEAN and lmx <= LSE_MAX, tag


def _check_grad(g, ref, tag):
    g = _f64(g)
    top = float(np.abs(ref).max(initial=0.0)) or 1.0
    err = np.abs(g - ref)
    print(f"[parity] {tag}: max {err.max(initial=0.0) / top:.2e} mean {err.mean() / top:.2e} of max|ref|",
          flush=True)
    assert err.max(initial=0.0) <= G_MAX * top and err.mean() <= G_MEAN * top, tag


def _draw(rng):
    H = int(rng.choice([1, 2, 3, 4, 6, 8]))
    divisors = [g for g in range(1, H + 1) if H % g == 0]
    return {
        "B": int(rng.integers(1, 3)),
        "H": H,
        "H_kv": int(rng.choice(divisors)),
        "N": int(rng.integers(1, 600)),
        "d": int(8 * rng.integers(1, 33)),
        "causal": bool(rng.integers(0, 2)),
        "scale": float(rng.choice([-1.0, 1.0]) * rng.uniform(0.02, 0.4)),
        "varlen": bool(rng.random() < 0.3),
        "bwd": bool(rng.random() < 1 / 3),
    }


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    rng = np.random.default_rng(7000 + case)
    c = _draw(rng)
    d, H, H_kv, causal = c["d"], c["H"], c["H_kv"], c["causal"]
    scale = float(np.float32(c["scale"]))
    variant = int(rng.integers(0, fa2.num_variants(d)))
    tag = f"case {case} {c} v{variant}"
    print(f"[case] {tag}", flush=True)
    if c["varlen"]:
        lengths = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 200, 256, 257, 511], size=int(rng.integers(1, 5)))]
        if sum(lengths) == 0:
            lengths.append(5)
        q, k, v, cu, _ = make_varlen(H, d, 7100 + case, lengths=lengths, H_kv=H_kv)
        o, l = fa2.fwd_varlen_gqa(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths), causal=causal,
                                  scale=scale, variant=variant)
        torch.cuda.synchronize()
        o_ref, l_ref = attention_varlen_gqa(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                            cu.numpy(), causal, scale)
        _check_fwd(o, l, o_ref, l_ref, tag)
        return
    q, k, v = make_qkv(c["B"], H, c["N"], d, 7200 + case, H_kv=H_kv)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = fa2.fwd_gqa(qd, kd, vd, causal=causal, scale=scale, variant=variant)
    torch.cuda.synchronize()
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    o_ref, l_ref = attention_gqa(qn, kn, vn, causal, scale)
    _check_fwd(o, l, o_ref, l_ref, tag)
    if c["bwd"]:
        gen = torch.Generator().manual_seed(7300 + case)
        do = torch.randn(q.shape, generator=gen).to(torch.bfloat16)
        dq, dk, dv = fa2.bwd(qd, kd, vd, o, l, do.to(DEV), causal=causal, scale=scale)
        torch.cuda.synchronize()
        refs = attention_backward_gqa(qn, kn, vn, do.double().numpy(), causal, scale)
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            _check_grad(g, ref, f"{tag} {name}")
