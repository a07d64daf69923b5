"""Host-side checks of the C ABI (no GPU needed; nothing here launches a kernel).

Every call below either fails validation before any HIP call, or (where the arguments are valid
and a launch would follow) runs only where no GPU is visible, so that the device query fails
first: the fake pointers are never handed to a kernel.

* libfa2.so loads and exports every function include/fa2.h declares;
* argument validation returns the documented status codes before any HIP call;
* the launch geometry agrees with the worked sizing example of the llm-infra-atlas page
  ("FlashAttention", section 4), stored in tests/golden/llm_infra_atlas_sizing.json.
"""
import ctypes
import json
import os
import re

import pytest

import exact_softmax_attention_amd as fa2
from exact_softmax_attention_amd import _lib
from synthetic import metric_flops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def _gpu_present():
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa2.load_library()
    names = _declared_functions()
    assert "fa2_fwd" in names and "fa2_fwd_varlen" in names
    for name in names:
        assert hasattr(lib, name), f"libfa2.so does not export {name}"
    # and the binding declares a signature for each of them
    assert set(names) == set(_lib._SIGNATURES)


def test_abi_version_and_status_strings():
    lib = fa2.load_library()
    assert lib.fa2_abi_version() == fa2.FA2_ABI_VERSION
    for code in list(fa2.STATUS) + [12345, -1]:
        s = lib.fa2_status_str(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_variants_listed():
    # A head dim that is not 64/128/256 runs on the next kernel width: same variants.
    for d, dpad in ((8, 64), (96, 128), (192, 256)):
        assert [fa2.variant_name(d, i) for i in range(fa2.num_variants(d))] == \
            [fa2.variant_name(dpad, i) for i in range(fa2.num_variants(dpad))]
    for d in (64, 128, 256):
        n = fa2.num_variants(d)
        assert n >= 1
        names = [fa2.variant_name(d, i) for i in range(n)]
        assert all(names) and len(set(names)) == n
        assert fa2.variant_name(d, n) == ""
    assert fa2.num_variants(100) == 0


def test_varlen_default_variant():
    # fa2_fwd_varlen runs the persistent d = 128 form at head dims 72..128, variant 0 elsewhere.
    persist = [fa2.variant_name(128, i) for i in range(fa2.num_variants(128))].index("d128_w8_bc64_persist")
    for d in (72, 96, 120, 128):
        assert fa2.varlen_default_variant(d) == persist, d
    for d in (8, 64, 136, 256, 100, 0, 264):
        assert fa2.varlen_default_variant(d) == 0, d


def test_geometry_matches_worked_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "llm_infra_atlas_sizing.json")))
    N, d, H, B = g["N"], g["head_dim"], g["heads"], g["batch"]
    # the page's tile arithmetic for its Br = Bc = 128
    assert (N // g["Br"], H, B) == tuple(g["grid"])
    assert N // g["Bc"] == g["kv_iterations"]
    assert g["Br"] * g["Bc"] * g["bytes_per_elem"] == g["S_block_bytes"]
    assert N * N * g["bytes_per_elem"] == g["S_head_bytes"]
    assert N * N * g["bytes_per_elem"] * H * B == g["S_all_heads_bytes"]
    # the library's geometry for the same problem: B*H*ceil(N/Br) workgroups
    for v in range(fa2.num_variants(d)):
        geo = fa2.geometry(B, H, N, d, causal=False, variant=v)
        br, bc = geo["block_rows"], geo["block_cols"]
        assert geo["num_workgroups"] == -(-N // br) * H * B
        if br == g["Br"]:
            assert geo["num_workgroups"] == g["grid"][0] * g["grid"][1] * g["grid"][2]
        assert geo["lds_bytes"] <= 160 * 1024
        # causal: the average number of key tiles a row block visits is about half of N/Bc
        tr = -(-N // br)
        visits = [min(N, (i + 1) * br) for i in range(tr)]
        avg = sum(-(-x // bc) for x in visits) / tr
        assert abs(avg / (N / bc) - 0.5) < 0.02


def test_geometry_errors():
    assert fa2.geometry(1, 1, 0, 64)["num_workgroups"] == 0
    for args, code in (((0, 1, 8, 64), 2), ((1, 0, 8, 64), 2), ((1, 1, -1, 64), 2), ((1, 1, 8, 100), 3)):
        with pytest.raises(fa2.Fa2Error) as e:
            fa2.geometry(*args)
        assert e.value.status == code
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.geometry(1 << 16, 1 << 10, 1 << 20, 128)
    assert e.value.status == 9


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, causal=0, scale=0.125, variant=0):
    return fa2.load_library().fa2_fwd_variant(q, k, v, o, lse, B, H, N, d, causal, scale, variant, None)


def _varlen(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, S=2, maxlen=16, T=32, H=1, d=64, causal=1,
            scale=0.125, variant=0):
    return fa2.load_library().fa2_fwd_varlen_variant(q, k, v, o, lse, cu, S, maxlen, T, H, d, causal, scale,
                                                     variant, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=-5), 2),
    (dict(d=100), 3), (dict(d=264), 3), (dict(d=512), 3), (dict(d=0), 3), (dict(d=4), 3),
    (dict(q=FAKE + 8), 4), (dict(o=FAKE + 2), 4), (dict(lse=FAKE + 2), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5), (dict(scale=-float("inf")), 5),
    (dict(variant=-1), 8), (dict(variant=99), 8),
    (dict(B=1 << 16, H=1 << 10, N=1 << 20, d=128), 9),
])
def test_fwd_validation(kwargs, code):
    assert _fwd(**kwargs) == code


def _fwd_plain(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, causal=0, scale=0.125):
    return fa2.load_library().fa2_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None)


def _varlen_plain(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, S=2, maxlen=16, T=32, H=1, d=64, causal=1,
                  scale=0.125):
    return fa2.load_library().fa2_fwd_varlen(q, k, v, o, lse, cu, S, maxlen, T, H, d, causal, scale, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=-1), 2),
    (dict(d=100), 3), (dict(d=0), 3), (dict(d=264), 3),
    (dict(q=FAKE + 2), 4), (dict(v=FAKE + 8), 4), (dict(lse=FAKE + 1), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5),
    (dict(B=1 << 16, H=1 << 10, N=1 << 20, d=128), 9),
])
def test_fwd_plain_entry_validation(kwargs, code):
    """fa2_fwd itself (the entry point with no variant argument) returns the header's codes."""
    assert _fwd_plain(**kwargs) == code


def test_fwd_plain_entry_empty():
    assert _fwd_plain(q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert _fwd_plain(q=None, k=None, v=None, o=None, lse=None, N=0, d=12) == 3


@pytest.mark.parametrize("kwargs,code", [
    (dict(cu=None), 1), (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(H=0), 2), (dict(S=-1), 2), (dict(maxlen=-1), 2), (dict(T=-1), 2),
    (dict(d=84), 3), (dict(d=512), 3), (dict(cu=FAKE + 2), 4), (dict(k=FAKE + 4), 4), (dict(o=FAKE + 8), 4),
    (dict(scale=float("nan")), 5), (dict(scale=-float("inf")), 5),
    (dict(S=1 << 20, maxlen=1 << 20, T=1 << 20, H=64), 9),
])
def test_varlen_plain_entry_validation(kwargs, code):
    """fa2_fwd_varlen itself returns the header's codes."""
    assert _varlen_plain(**kwargs) == code


def test_varlen_plain_entry_empty():
    assert _varlen_plain(S=0, cu=None, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _varlen_plain(T=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _varlen_plain(maxlen=0, q=None, k=None, v=None, o=None, lse=None) == 0


def test_status_string_states_the_head_dim_rule():
    """The text of FA2_ERR_UNSUPPORTED_HEADDIM says what the header's rule says: any multiple
    of 8 from 8 to 256, for the forward and the backward alike."""
    text = fa2.load_library().fa2_status_str(3).decode()
    assert "multiple of 8" in text and "8 to 256" in text and "backward" in text
    header = open(HEADER).read()
    assert "FA2_ERR_UNSUPPORTED_HEADDIM = 3, /* d not a multiple of 8 in [8, 256] */" in header
    # and the rule itself: 8..256 step 8 pass validation, everything else fails it
    for d in range(0, 300):
        want = 3 if (d < 8 or d > 256 or d % 8) else 0
        got = _fwd_plain(N=0, q=None, k=None, v=None, o=None, lse=None, d=d)
        assert got == want, d
        gotb = _bwd(N=0, d=d, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                    delta=None)
        assert gotb == want, d


def test_fwd_empty_is_ok_without_pointers():
    assert _fwd(q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert _fwd(q=None, k=None, v=None, o=None, lse=None, N=0, d=100) == 3


@pytest.mark.parametrize("kwargs,code", [
    (dict(cu=None), 1), (dict(q=None), 1), (dict(lse=None), 1),
    (dict(H=0), 2), (dict(S=-1), 2), (dict(maxlen=-1), 2), (dict(T=-1), 2),
    (dict(d=84), 3), (dict(cu=FAKE + 2), 4), (dict(k=FAKE + 4), 4),
    (dict(scale=float("nan")), 5), (dict(variant=999), 8),
    (dict(S=1 << 20, maxlen=1 << 20, T=1 << 20, H=64), 9),
])
def test_varlen_validation(kwargs, code):
    assert _varlen(**kwargs) == code


def test_varlen_empty_is_ok():
    assert _varlen(S=0, cu=None, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _varlen(T=0, q=None, k=None, v=None, o=None, lse=None) == 0


def _gqa(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=8, H_kv=2, N=16, d=128, causal=1, scale=0.125,
         variant=0):
    return fa2.load_library().fa2_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, variant, None)


def _varlen_gqa(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, S=2, maxlen=16, T=32, H=8, H_kv=4, d=64,
                causal=1, scale=0.125, variant=0):
    return fa2.load_library().fa2_fwd_varlen_gqa(q, k, v, o, lse, cu, S, maxlen, T, H, H_kv, d, causal, scale,
                                                 variant, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(H_kv=0), 2), (dict(H_kv=-2), 2), (dict(H_kv=3), 2), (dict(H_kv=16), 2), (dict(H=0), 2),
    (dict(k=None), 1), (dict(v=FAKE + 4), 4), (dict(d=36), 3), (dict(variant=77), 8),
    (dict(scale=float("nan")), 5),
])
def test_gqa_validation(kwargs, code):
    assert _gqa(**kwargs) == code


@pytest.mark.parametrize("kwargs,code", [
    (dict(H_kv=0), 2), (dict(H_kv=3), 2), (dict(cu=None), 1), (dict(d=97), 3), (dict(variant=-1), 8),
])
def test_varlen_gqa_validation(kwargs, code):
    assert _varlen_gqa(**kwargs) == code


def test_gqa_empty_is_ok():
    assert _gqa(q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert _varlen_gqa(T=0, q=None, k=None, v=None, o=None, lse=None) == 0


def _bwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE, B=1, H=4,
         H_kv=2, N=64, d=128, causal=1, scale=0.088):
    return fa2.load_library().fa2_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale,
                                       None)


def _bwd_varlen(cu=FAKE, S=2, maxlen=16, T=32, H=4, H_kv=4, d=64, causal=0, scale=0.125, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE)
    p.update(ptrs)
    return fa2.load_library().fa2_bwd_varlen(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"],
                                              p["dv"], p["delta"], cu, S, maxlen, T, H, H_kv, d, causal, scale,
                                              None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1), (dict(delta=None), 1),
    (dict(B=0), 2), (dict(H_kv=3), 2), (dict(H_kv=0), 2), (dict(N=-1), 2),
    (dict(d=100), 3), (dict(d=264), 3), (dict(d=4), 3), (dict(dq=FAKE + 8), 4), (dict(delta=FAKE + 2), 4), (dict(o=FAKE + 4), 4),
    (dict(scale=float("nan")), 5), (dict(N=1 << 30, H=64, H_kv=64), 9),
])
def test_bwd_validation(kwargs, code):
    assert _bwd(**kwargs) == code


@pytest.mark.parametrize("kwargs,code", [
    (dict(cu=None), 1), (dict(dv=None), 1), (dict(H_kv=3), 2), (dict(S=-1), 2), (dict(d=36), 3),
    (dict(cu=FAKE + 2), 4), (dict(scale=float("inf")), 5),
])
def test_bwd_varlen_validation(kwargs, code):
    assert _bwd_varlen(**kwargs) == code


def test_bwd_empty_is_ok():
    none = dict(q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None, delta=None)
    assert _bwd(N=0, **none) == 0
    assert _bwd_varlen(T=0, cu=None, **none) == 0


def _bwd_ws(ws=FAKE, nbytes=1 << 40, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
            delta=FAKE, B=1, H=8, H_kv=2, N=64, d=128, causal=1, scale=0.088):
    return fa2.load_library().fa2_bwd_ws(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale,
                                          ws, nbytes, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(ws=None), 1), (dict(ws=FAKE + 8), 4), (dict(nbytes=0), 10), (dict(nbytes=-1), 10),
    (dict(q=None), 1), (dict(H_kv=3), 2), (dict(d=100), 3), (dict(dk=FAKE + 2), 4),
    (dict(scale=float("nan")), 5),
])
def test_bwd_ws_validation(kwargs, code):
    """Every case fails before any launch: the workspace is needed for this shape (H=8 over
    H_kv=2, 64 keys) and checked after the tensors."""
    assert _bwd_ws(**kwargs) == code


def test_bwd_workspace_bytes():
    """Query-head splits: the smallest divisor S of g that gives the dK/dV kernel (one wave
    per 32 keys of each key/value head and split) its waves per SIMD on 1024 SIMDs (two at
    d = 128, three at d = 64; four times as many when causal), else g; S * 2 * B * H_kv * N * d
    fp32 values when S > 1."""
    f = fa2.load_library().fa2_bwd_workspace_bytes
    for causal in (0, 1):
        assert f(1, 16, 16, 16384, 128, causal) == 0                   # no groups
        assert f(1, 8, 2, 300, 64, causal) == 4 * 2 * 1 * 2 * 300 * 64 * 4  # S = g = 4
    assert f(1, 16, 2, 16384, 128, 0) == 2 * 2 * 1 * 2 * 16384 * 128 * 4   # 1024 waves -> S = 2
    assert f(1, 16, 2, 16384, 128, 1) == 8 * 2 * 1 * 2 * 16384 * 128 * 4   # causal: S = 8
    assert f(1, 16, 1, 16384, 128, 0) == 4 * 2 * 1 * 1 * 16384 * 128 * 4   # 512 waves -> S = 4
    assert f(1, 16, 1, 16384, 128, 1) == 16 * 2 * 1 * 1 * 16384 * 128 * 4
    assert f(8, 16, 2, 2048, 128, 0) == 2 * 2 * 8 * 2 * 2048 * 128 * 4
    assert f(16, 16, 2, 4096, 128, 0) == 0                               # 4096 waves already
    assert f(16, 16, 2, 4096, 128, 1) == 2 * 2 * 16 * 2 * 4096 * 128 * 4
    assert f(1, 12, 4, 1000, 96, 0) == 3 * 2 * 1 * 4 * 1000 * 96 * 4       # g = 3, padded d
    for bad in ((0, 8, 2, 64, 64), (1, 6, 4, 64, 64), (1, 8, 2, 0, 64), (1, 8, 2, 64, 100), (1, 8, 0, 64, 64)):
        assert f(*bad, 1) == 0


def _chunk(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, H_kv=2, Nq=16, Nk=32, d=64, causal=1, diag=0,
           scale=0.125, variant=0):
    return fa2.load_library().fa2_fwd_chunk(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, causal, diag, scale, variant,
                                            None)


def _splitkv(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, H_kv=2, Nq=16, Nk=640, d=128, causal=1, diag=0,
             scale=0.088, S=4, op=FAKE, lp=FAKE, variant=0):
    return fa2.load_library().fa2_fwd_splitkv(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, causal, diag, scale, S, op, lp,
                                              variant, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(S=0), 2), (dict(S=-3), 2), (dict(op=None), 1), (dict(lp=None), 1), (dict(op=FAKE + 8), 4),
    (dict(lp=FAKE + 1), 4), (dict(S=70000), 9), (dict(H_kv=3), 2), (dict(d=512), 3), (dict(variant=-2), 8),
])
def test_splitkv_validation(kwargs, code):
    assert _splitkv(**kwargs) == code


@pytest.mark.skipif(_gpu_present(), reason="valid calls would launch on fake pointers where a GPU is visible")
def test_splitkv_workspace_unused_without_split():
    # One split, or no keys: the workspace is not needed; validation passes and the call
    # stops at the device query (no GPU here).
    assert _splitkv(S=1, op=None, lp=None) == 6
    assert _splitkv(Nk=0, k=None, v=None, op=None, lp=None) == 6


def _noalloc(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, H_kv=2, Nq=16, Nk=640, d=128, causal=1, diag=0,
             scale=0.088, S=4, variant=0):
    return fa2.load_library().fa2_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, causal, diag, scale,
                                                      S, variant, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(S=0), 2), (dict(S=-3), 2), (dict(H_kv=3), 2), (dict(Nq=-1), 2), (dict(q=None), 1), (dict(lse=None), 1),
    (dict(d=81), 3), (dict(d=512), 3), (dict(o=FAKE + 2), 4), (dict(lse=FAKE + 1), 4),
    (dict(scale=float("nan")), 5), (dict(variant=50), 8), (dict(S=70000), 9),
    # 8 pieces of 32 x 4096 rows at d = 128 need 8 * 131072 * 260 B = 260 MiB > 32 MiB
    (dict(H=32, H_kv=32, Nq=4096, Nk=8192, S=8), 10),
])
def test_noalloc_validation(kwargs, code):
    """fa2_fwd_splitkv_noalloc returns the header's codes before any HIP call, including
    FA2_ERR_SCRATCH_TOO_SMALL when the partials would not fit the static scratch."""
    assert _noalloc(**kwargs) == code


def test_noalloc_scratch_rule():
    # the limit is the header's FA2_STATIC_SCRATCH_BYTES; one piece needs no scratch at all
    header = open(HEADER).read()
    assert "#define FA2_STATIC_SCRATCH_BYTES (32u << 20)" in header
    assert _lib.FA2_STATIC_SCRATCH_BYTES == 32 << 20
    assert _noalloc(Nq=0, q=None, k=None, v=None, o=None, lse=None) == 0


def _merge(op=FAKE, lp=FAKE, S=2, rows=100, d=128, o=FAKE, lse=FAKE):
    return fa2.load_library().fa2_lse_merge(op, lp, S, rows, d, o, lse, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(Nq=-1), 2), (dict(Nk=-1), 2), (dict(H_kv=3), 2), (dict(diag=(1 << 30) + 1), 2),
    (dict(diag=-(1 << 30) - 1), 2), (dict(q=None), 1), (dict(k=None), 1), (dict(d=81), 3),
    (dict(o=FAKE + 2), 4), (dict(variant=50), 8), (dict(scale=float("nan")), 5),
    (dict(B=1 << 10, H=1 << 10, Nq=1 << 12), 9),
])
def test_chunk_validation(kwargs, code):
    assert _chunk(**kwargs) == code


def test_chunk_empty():
    assert _chunk(Nq=0, q=None, k=None, v=None, o=None, lse=None) == 0


@pytest.mark.skipif(_gpu_present(), reason="valid calls would launch on fake pointers where a GPU is visible")
def test_chunk_no_keys_passes_validation():
    # N_k == 0: k and v may be NULL; with valid q/o/lse the call passes validation and
    # stops at the device query (no GPU here).
    assert _chunk(Nk=0, k=None, v=None) == 6


@pytest.mark.parametrize("kwargs,code", [
    (dict(S=0), 2), (dict(rows=-1), 2), (dict(d=100), 3), (dict(op=None), 1), (dict(lse=None), 1),
    (dict(op=FAKE + 8), 4), (dict(lp=FAKE + 2), 4), (dict(o=FAKE + 4), 4),
])
def test_merge_validation(kwargs, code):
    assert _merge(**kwargs) == code


def test_merge_empty_is_ok():
    assert _merge(rows=0, op=None, lp=None, o=None, lse=None) == 0


@pytest.mark.skipif(_gpu_present(), reason="only meaningful where no GPU is visible")
def test_no_device_reported():
    # Valid arguments: validation passes, then the device query fails before any launch.
    assert _fwd() == 6
    assert _fwd_plain() == 6
    assert _varlen() == 6
    assert _varlen_plain() == 6
    assert _gqa() == 6
    assert _varlen_gqa() == 6
    assert _bwd() == 6
    assert _bwd_varlen() == 6
    assert _chunk() == 6
    assert _merge() == 6
    assert _splitkv() == 6
    assert _noalloc() == 6
    assert _noalloc(S=1) == 6


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa2.fwd(q, q, q)
    with pytest.raises(ValueError):
        fa2.fwd_gqa(q, q, q)


def test_metric_flops():
    # 4*B*H*N^2*d, halved for causal (paper-graph-ui "Evaluation Methodology", Metrics)
    assert metric_flops(1, 16, 16384, 128, True) == 2 * 16 * 16384 ** 2 * 128
    assert metric_flops(8, 16, 2048, 128, False) == 4 * 8 * 16 * 2048 ** 2 * 128


def test_binding_rejects_tensors_on_different_devices():
    import torch
    a = torch.zeros(2)
    _lib._same_device(a, torch.zeros(3))                       # one device: fine
    with pytest.raises(ValueError, match="one device"):
        _lib._same_device(a, torch.zeros(2, device="meta"))


def test_autograd_wrapper_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    import exact_softmax_attention_amd as fa2
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa2.attention(q, q, q)
