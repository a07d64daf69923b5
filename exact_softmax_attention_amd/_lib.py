"""ctypes marshalling for libfa2.so (see include/fa2.h for the C ABI)."""
from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
FA2_ABI_VERSION = 1

STATUS = {
    0: "FA2_OK",
    1: "FA2_ERR_NULL_PTR",
    2: "FA2_ERR_BAD_SHAPE",
    3: "FA2_ERR_UNSUPPORTED_HEADDIM",
    4: "FA2_ERR_MISALIGNED",
    5: "FA2_ERR_BAD_SCALE",
    6: "FA2_ERR_NO_DEVICE",
    7: "FA2_ERR_LAUNCH",
    8: "FA2_ERR_BAD_VARIANT",
    9: "FA2_ERR_TOO_LARGE",
    10: "FA2_ERR_SCRATCH_TOO_SMALL",
}

FA2_STATIC_SCRATCH_BYTES = 32 << 20

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float

_SIGNATURES = {
    "fa2_fwd": ([_c_void_p] * 5 + [_c_int] * 5 + [_c_float, _c_void_p], _c_int),
    "fa2_fwd_variant": ([_c_void_p] * 5 + [_c_int] * 5 + [_c_float, _c_int, _c_void_p], _c_int),
    "fa2_fwd_varlen": ([_c_void_p] * 6 + [_c_int] * 6 + [_c_float, _c_void_p], _c_int),
    "fa2_fwd_varlen_variant": ([_c_void_p] * 6 + [_c_int] * 6 + [_c_float, _c_int, _c_void_p], _c_int),
    "fa2_fwd_gqa": ([_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_int, _c_void_p], _c_int),
    "fa2_fwd_varlen_gqa": ([_c_void_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_void_p], _c_int),
    "fa2_fwd_chunk": ([_c_void_p] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_void_p], _c_int),
    "fa2_fwd_splitkv": ([_c_void_p] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_void_p, _c_void_p, _c_int,
                                                            _c_void_p], _c_int),
    "fa2_fwd_splitkv_noalloc": ([_c_void_p] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_int, _c_void_p], _c_int),
    "fa2_lse_merge": ([_c_void_p, _c_void_p, _c_int, ctypes.c_longlong, _c_int, _c_void_p, _c_void_p, _c_void_p],
                      _c_int),
    "fa2_bwd": ([_c_void_p] * 10 + [_c_int] * 6 + [_c_float, _c_void_p], _c_int),
    "fa2_bwd_ws": ([_c_void_p] * 10 + [_c_int] * 6 + [_c_float, _c_void_p, ctypes.c_longlong, _c_void_p], _c_int),
    "fa2_bwd_workspace_bytes": ([_c_int] * 6, ctypes.c_longlong),
    "fa2_bwd_varlen_ws": ([_c_void_p] * 11 + [_c_int] * 7 + [_c_float, _c_void_p, ctypes.c_longlong, _c_void_p],
                          _c_int),
    "fa2_bwd_varlen_workspace_bytes": ([_c_int] * 7, ctypes.c_longlong),
    "fa2_bwd_varlen": ([_c_void_p] * 11 + [_c_int] * 7 + [_c_float, _c_void_p], _c_int),
    "fa2_num_variants": ([_c_int], _c_int),
    "fa2_fwd_geometry": ([_c_int] * 6 + [ctypes.POINTER(_c_int)] * 4, _c_int),
    "fa2_status_str": ([_c_int], ctypes.c_char_p),
    "fa2_variant_name": ([_c_int, _c_int], ctypes.c_char_p),
    "fa2_fwd_varlen_default_variant": ([_c_int], _c_int),
    "fa2_abi_version": ([], _c_int),
}

_LIB = None


class Fa2Error(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(PKG_DIR, "libfa2.so")


def load_library():
    """Load libfa2.so (built in-tree). Raises loudly if it is missing: there is no fallback."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run `python -m exact_softmax_attention_amd.build` "
                              "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(path)
        for name, (argtypes, restype) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = restype
        if lib.fa2_abi_version() != FA2_ABI_VERSION:
            raise ImportError(f"libfa2.so ABI {lib.fa2_abi_version()} != binding ABI {FA2_ABI_VERSION}")
        _LIB = lib
    return _LIB


def _check(status: int):
    if status != 0:
        raise Fa2Error(status, load_library().fa2_status_str(status).decode())


def num_variants(d: int) -> int:
    return load_library().fa2_num_variants(d)


def variant_name(d: int, variant: int) -> str:
    return load_library().fa2_variant_name(d, variant).decode()


def varlen_default_variant(d: int) -> int:
    """Index of the variant ``fa2_fwd_varlen`` runs for head dimension d."""
    return load_library().fa2_fwd_varlen_default_variant(d)


def geometry(B: int, H: int, N: int, d: int, causal: bool = False, variant: int = 0) -> dict:
    """Launch geometry computed on the host (no GPU needed)."""
    out = [_c_int(0) for _ in range(4)]
    _check(load_library().fa2_fwd_geometry(B, H, N, d, int(causal), variant, *[ctypes.byref(x) for x in out]))
    return {"num_workgroups": out[0].value, "block_rows": out[1].value,
            "block_cols": out[2].value, "lds_bytes": out[3].value}


def _torch():
    import torch
    return torch


def _stream_ptr(dev) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(dev).cuda_stream)


def _check_tensor(name, t, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU (HIP) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*tensors):
    """Every tensor of one call must live on the device the kernels are launched on."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors of a call must be on one device; got {dev} and {t.device}")


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
        variant: int | None = None):
    """O, LSE = softmax(scale * q k^T [causal mask]) v for bf16 [B, H, N, d] tensors.

    Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N]); ``out``/``lse`` may be given
    preallocated. Enqueued on torch's current stream of q's device. Without ``variant`` the
    call goes to ``fa2_fwd`` (the default kernel); with one, to ``fa2_fwd_variant``.
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    if out.shape != q.shape or tuple(lse.shape) != (B, H, N) or out.device != q.device or lse.device != q.device:
        raise ValueError("out/lse shape or device mismatch")
    _same_device(q, k, v, out, lse)
    lib = load_library()
    with torch.cuda.device(q.device):
        if variant is None:
            st = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, H, N, d, int(bool(causal)), float(scale), _stream_ptr(q.device))
        else:
            st = lib.fa2_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, int(bool(causal)), float(scale), int(variant),
                                     _stream_ptr(q.device))
    _check(st)
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
               out=None, lse=None, variant: int | None = None):
    """Packed variable-length forward over bf16 [H, T, d] tensors.

    ``cu_seqlens`` is an int32 GPU tensor [num_seqs + 1]; sequence s owns tokens
    [cu[s], cu[s+1]). Returns (o bf16 [H, T, d], lse fp32 [H, T]). Without ``variant`` the
    call goes to ``fa2_fwd_varlen``; with one, to ``fa2_fwd_varlen_variant``.
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 3)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    H, T, d = q.shape
    num_seqs = cu_seqlens.numel() - 1
    if num_seqs < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    if out.shape != q.shape or tuple(lse.shape) != (H, T):
        raise ValueError("out/lse shape mismatch")
    _same_device(q, k, v, cu_seqlens, out, lse)
    lib = load_library()
    with torch.cuda.device(q.device):
        if variant is None:
            st = lib.fa2_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    cu_seqlens.data_ptr(), num_seqs, int(max_seqlen), T, H, d,
                                    int(bool(causal)), float(scale), _stream_ptr(q.device))
        else:
            st = lib.fa2_fwd_varlen_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            lse.data_ptr(), cu_seqlens.data_ptr(), num_seqs, int(max_seqlen), T, H,
                                            d, int(bool(causal)), float(scale), int(variant),
                                            _stream_ptr(q.device))
    _check(st)
    return out, lse


def fwd_gqa(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, variant: int = 0):
    """Grouped-/multi-query forward: q bf16 [B, H, N, d]; k, v bf16 [B, H_kv, N, d].

    Query head h attends with key/value head h // (H // H_kv); H_kv must divide H.
    Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N]).
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 4)
    if k.shape != v.shape:
        raise ValueError(f"k, v shapes differ: {tuple(k.shape)} {tuple(v.shape)}")
    B, H, N, d = q.shape
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    H_kv = k.shape[1]
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    if out.shape != q.shape or tuple(lse.shape) != (B, H, N) or out.device != q.device or lse.device != q.device:
        raise ValueError("out/lse shape or device mismatch")
    _same_device(q, k, v, out, lse)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa2_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, H, H_kv, N, d, int(bool(causal)), float(scale), int(variant),
                             _stream_ptr(q.device))
    _check(st)
    return out, lse


def fwd_varlen_gqa(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
                   out=None, lse=None, variant: int | None = None):
    """Packed variable-length grouped-query forward: q [H, T, d], k/v [H_kv, T, d] bf16.

    Without ``variant`` the call runs the variant ``fa2_fwd_varlen`` picks for d
    (``varlen_default_variant``)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 3)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k/v shapes do not match q")
    H, T, d = q.shape
    H_kv = k.shape[0]
    num_seqs = cu_seqlens.numel() - 1
    if num_seqs < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if variant is None:
        variant = varlen_default_variant(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    if out.shape != q.shape or tuple(lse.shape) != (H, T):
        raise ValueError("out/lse shape mismatch")
    _same_device(q, k, v, cu_seqlens, out, lse)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa2_fwd_varlen_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    cu_seqlens.data_ptr(), num_seqs, int(max_seqlen), T, H, H_kv, d,
                                    int(bool(causal)), float(scale), int(variant), _stream_ptr(q.device))
    _check(st)
    return out, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, delta=None, split: bool = True):
    """Gradients (dq, dk, dv) of the forward for upstream gradient ``dout``.

    q, o, dout: bf16 [B, H, N, d]; k, v: bf16 [B, H_kv, N, d] (H_kv divides H); lse: fp32
    [B, H, N] from the forward with the same ``scale``. ``delta`` (fp32 [B, H, N]) is the
    scratch buffer for D = rowsum(dout * o); outputs and scratch are allocated when not given.
    With grouped- or multi-query heads and ``split`` (the default) the call goes to
    fa2_bwd_ws, which spreads each group's query heads over several dK/dV workgroups, with
    the workspace it asks for allocated here; ``split=False`` calls fa2_bwd.
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or \
            (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError("q/o/dout [B,H,N,d], k/v [B,H_kv,N,d], lse [B,H,N] shapes do not match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, torch.bfloat16, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(ref.shape)}")
    _check_tensor("delta", delta, torch.float32, 3)
    if tuple(delta.shape) != (B, H, N):
        raise ValueError("delta must be [B, H, N]")
    _same_device(q, k, v, o, lse, dout, dq, dk, dv, delta)
    lib = load_library()
    ws_bytes = lib.fa2_bwd_workspace_bytes(B, H, H_kv, N, d, int(bool(causal))) if split and H_kv != H else 0
    with torch.cuda.device(q.device):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                B, H, H_kv, N, d, int(bool(causal)), float(scale))
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            st = lib.fa2_bwd_ws(*args, ws.data_ptr(), ws_bytes, _stream_ptr(q.device))
        else:
            st = lib.fa2_bwd(*args, _stream_ptr(q.device))
    _check(st)
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen: int, causal: bool = False,
               scale: float | None = None, dq=None, dk=None, dv=None, delta=None, split: bool = True):
    """Packed variable-length backward: q, o, dout [H, T, d]; k, v [H_kv, T, d]; lse [H, T].
    Grouped heads with ``split`` go to fa2_bwd_varlen_ws (workspace allocated here), as in
    ``bwd``."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    H, T, d = q.shape
    H_kv = k.shape[0]
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or k.shape[1:] != q.shape[1:] \
            or tuple(lse.shape) != (H, T):
        raise ValueError("q/o/dout [H,T,d], k/v [H_kv,T,d], lse [H,T] shapes do not match")
    num_seqs = cu_seqlens.numel() - 1
    if num_seqs < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((H, T), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, torch.bfloat16, 3)
        if t.shape != ref.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(ref.shape)}")
    _check_tensor("delta", delta, torch.float32, 2)
    if tuple(delta.shape) != (H, T):
        raise ValueError("delta must be [H, T]")
    _same_device(q, k, v, o, lse, dout, cu_seqlens, dq, dk, dv, delta)
    lib = load_library()
    ws_bytes = (lib.fa2_bwd_varlen_workspace_bytes(num_seqs, int(max_seqlen), T, H, H_kv, d, int(bool(causal)))
                if split and H_kv != H else 0)
    with torch.cuda.device(q.device):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                cu_seqlens.data_ptr(), num_seqs, int(max_seqlen), T, H, H_kv, d,
                int(bool(causal)), float(scale))
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            st = lib.fa2_bwd_varlen_ws(*args, ws.data_ptr(), ws_bytes, _stream_ptr(q.device))
        else:
            st = lib.fa2_bwd_varlen(*args, _stream_ptr(q.device))
    _check(st)
    return dq, dk, dv


def fwd_chunk(q, k, v, causal: bool = False, diag: int = 0, scale: float | None = None, out=None, lse=None,
              variant: int = 0):
    """Forward of q bf16 [B, H, N_q, d] against one key/value chunk k, v bf16 [B, H_kv, N_k, d].

    Causal: query i may attend key j iff j <= i + diag. Rows with no allowed key get O = 0,
    LSE = -inf. Returns (o bf16 [B, H, N_q, d], lse fp32 [B, H, N_q]).
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 4)
    if k.shape != v.shape:
        raise ValueError("k, v shapes differ")
    B, H, N_q, d = q.shape
    H_kv, N_k = k.shape[1], k.shape[2]
    if (k.shape[0], k.shape[3]) != (B, d):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    if out.shape != q.shape or tuple(lse.shape) != (B, H, N_q):
        raise ValueError("out/lse shape mismatch")
    _same_device(q, k, v, out, lse)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa2_fwd_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, H_kv, N_q, N_k, d, int(bool(causal)), int(diag), float(scale), int(variant),
                               _stream_ptr(q.device))
    _check(st)
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse=None):
    """Merge partial results: o_parts bf16 [S, ..., d], lse_parts fp32 [S, ...] (same leading
    shape) -> (o bf16 [..., d], lse fp32 [...]) with LSE = log sum exp(LSE_s) and
    O = sum exp(LSE_s - LSE) O_s."""
    torch = _torch()
    _check_tensor("o_parts", o_parts, torch.bfloat16, o_parts.dim())
    _check_tensor("lse_parts", lse_parts, torch.float32, lse_parts.dim())
    if o_parts.dim() < 2 or tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape):
        raise ValueError("o_parts must be [S, ..., d] with lse_parts [S, ...]")
    S, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts.numel() // S if S else 0
    out = torch.empty(o_parts.shape[1:], dtype=torch.bfloat16, device=o_parts.device) if out is None else out
    lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device) if lse is None else lse
    _check_tensor("out", out, torch.bfloat16, out.dim())
    _check_tensor("lse", lse, torch.float32, lse.dim())
    if tuple(out.shape) != tuple(o_parts.shape[1:]) or tuple(lse.shape) != tuple(lse_parts.shape[1:]):
        raise ValueError("out/lse shape mismatch")
    _same_device(o_parts, lse_parts, out, lse)
    lib = load_library()
    with torch.cuda.device(o_parts.device):
        st = lib.fa2_lse_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, rows, d, out.data_ptr(), lse.data_ptr(),
                               _stream_ptr(o_parts.device))
    _check(st)
    return out, lse


def fwd_splitkv(q, k, v, num_splits: int, causal: bool = False, diag: int = 0, scale: float | None = None,
                out=None, lse=None, o_parts=None, lse_parts=None, variant: int = 0):
    """``fwd_chunk`` with the keys split into up to ``num_splits`` pieces computed in one launch
    and merged by LSE. ``o_parts`` (bf16 [S, B, H, N_q, d]) and ``lse_parts`` (fp32
    [S, B, H, N_q]) are the workspace; allocated when not given."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 4)
    if k.shape != v.shape:
        raise ValueError("k, v shapes differ")
    B, H, N_q, d = q.shape
    H_kv, N_k = k.shape[1], k.shape[2]
    if (k.shape[0], k.shape[3]) != (B, d):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    S = int(num_splits)
    if S < 1:
        raise ValueError("num_splits must be >= 1")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device) if lse is None else lse
    if o_parts is None:
        o_parts = torch.empty((S, B, H, N_q, d), dtype=torch.bfloat16, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((S, B, H, N_q), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    _check_tensor("o_parts", o_parts, torch.bfloat16, 5)
    _check_tensor("lse_parts", lse_parts, torch.float32, 4)
    if out.shape != q.shape or tuple(lse.shape) != (B, H, N_q) or tuple(o_parts.shape) != (S, B, H, N_q, d) \
            or tuple(lse_parts.shape) != (S, B, H, N_q):
        raise ValueError("out/lse/o_parts/lse_parts shape mismatch")
    _same_device(q, k, v, out, lse, o_parts, lse_parts)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa2_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 B, H, H_kv, N_q, N_k, d, int(bool(causal)), int(diag), float(scale), S,
                                 o_parts.data_ptr(), lse_parts.data_ptr(), int(variant), _stream_ptr(q.device))
    _check(st)
    return out, lse
