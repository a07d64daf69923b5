"""Property tests of the host-side validation of fa2_fwd_gqa and fa2_bwd (no GPU needed).

For random argument combinations the status of each call must equal the one the rules of
include/fa2.h give, restated here independently and checked in the header's order: shape,
empty input, null pointers, head dimension, alignment, scale, variant, size limits; a call
that passes them all reaches the device query and, with no GPU visible, returns
FA2_ERR_NO_DEVICE. Fake pointer values are only ever passed where no GPU is visible.
"""
import ctypes
import math

import pytest
from hypothesis import given, settings, strategies as st

import exact_softmax_attention_amd as fa2

INT_MAX = 2 ** 31 - 1
BASE = 1 << 20
NAMES = ("q", "k", "v", "o", "lse")


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _expected(B, H, H_kv, N, d, scale, variant, null, misalign, n_variants):
    if B <= 0 or H <= 0 or H_kv <= 0 or H % H_kv != 0 or N < 0:
        return 2
    head_ok = 8 <= d <= 256 and d % 8 == 0
    if N == 0:
        return 0 if head_ok else 3
    if null is not None:
        return 1
    if not head_ok:
        return 3
    if misalign is not None:
        return 4
    if not math.isfinite(scale):
        return 5
    if not 0 <= variant < n_variants:
        return 8
    if B * H * N > INT_MAX or 2 * N + 1024 > INT_MAX:
        return 9
    return 6


@pytest.mark.skipif(_gpu_present(), reason="valid calls would launch on fake pointers where a GPU is visible")
@settings(max_examples=400, deadline=None)
@given(B=st.integers(-1, 5), H=st.integers(-1, 17), H_kv=st.integers(-1, 17),
       N=st.one_of(st.integers(-2, 5000), st.sampled_from([2 ** 20, 2 ** 27, 2 ** 30, INT_MAX])),
       d=st.one_of(st.sampled_from([64, 128, 256, 8, 96, 248]), st.integers(-8, 300)),
       scale=st.sampled_from([0.125, -0.5, 0.0, 1e30, float("inf"), float("nan")]),
       variant=st.integers(-1, 9), null=st.sampled_from((None,) + NAMES),
       misalign=st.sampled_from((None,) + NAMES))
def test_fwd_gqa_status_matches_the_header_rules(B, H, H_kv, N, d, scale, variant, null, misalign):
    lib = fa2.load_library()
    ptr = {}
    for i, name in enumerate(NAMES):
        addr = BASE + i * (1 << 12)
        if name == misalign:
            addr += 2 if name == "lse" else 8
        ptr[name] = None if name == null else ctypes.c_void_p(addr)
    n_variants = lib.fa2_num_variants(d)
    got = lib.fa2_fwd_gqa(ptr["q"], ptr["k"], ptr["v"], ptr["o"], ptr["lse"], B, H, H_kv, N, d, 1,
                          scale, variant, None)
    assert got == _expected(B, H, H_kv, N, d, scale, variant, null, misalign, n_variants)


BWD_NAMES = ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta")


def _expected_bwd(B, H, H_kv, N, d, scale, null, misalign):
    if B <= 0 or H <= 0 or H_kv <= 0 or H % H_kv != 0 or N < 0:
        return 2
    head_ok = 8 <= d <= 256 and d % 8 == 0
    if N == 0:
        return 0 if head_ok else 3
    if null is not None:
        return 1
    if not head_ok:
        return 3
    if misalign is not None:
        return 4
    if not math.isfinite(scale):
        return 5
    if (N + 127) // 128 * B * H > INT_MAX or B * H * N > INT_MAX:
        return 9
    return 6


@pytest.mark.skipif(_gpu_present(), reason="valid calls would launch on fake pointers where a GPU is visible")
@settings(max_examples=300, deadline=None)
@given(B=st.integers(-1, 5), H=st.integers(-1, 17), H_kv=st.integers(-1, 17),
       N=st.one_of(st.integers(-2, 5000), st.sampled_from([2 ** 20, 2 ** 27, INT_MAX])),
       d=st.one_of(st.sampled_from([64, 128, 256, 8, 96, 248]), st.integers(-8, 300)),
       scale=st.sampled_from([0.125, -0.5, 0.0, float("inf"), float("nan")]),
       null=st.sampled_from((None,) + BWD_NAMES), misalign=st.sampled_from((None,) + BWD_NAMES))
def test_bwd_status_matches_the_header_rules(B, H, H_kv, N, d, scale, null, misalign):
    lib = fa2.load_library()
    ptr = {}
    for i, name in enumerate(BWD_NAMES):
        addr = BASE + i * (1 << 12)
        if name == misalign:
            addr += 2 if name in ("lse", "delta") else 8
        ptr[name] = None if name == null else ctypes.c_void_p(addr)
    got = lib.fa2_bwd(*[ptr[n] for n in BWD_NAMES], B, H, H_kv, N, d, 1, scale, None)
    assert got == _expected_bwd(B, H, H_kv, N, d, scale, null, misalign)
