"""ctypes binding of the C ABI in include/fa.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``lib/libfa.so``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing, or a tensor is not
on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_LAUNCH",
    "FA_ERR_ALIGNMENT", "FA_ERR_TOO_LARGE", "FA_DTYPE_FP32", "FA_DTYPE_BF16", "FaError", "library_path", "lib",
    "forward", "backward", "backward_workspace_size", "backward_workspace", "workspace_delta",
    "backward_preprocess", "backward_dkdv", "backward_dq", "status_string", "version",
    "lse_merge", "decode", "decode_splits", "decode_workspace_size", "forward_merge", "backward_noalloc",
]

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_LAUNCH = 4
FA_ERR_ALIGNMENT = 5
FA_ERR_TOO_LARGE = 6
FA_DTYPE_FP32 = 0
FA_DTYPE_BF16 = 1

_DTYPES = {torch.float32: FA_DTYPE_FP32, torch.bfloat16: FA_DTYPE_BF16}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libfa.so")


def lib() -> ctypes.CDLL:
    """Load libfa.so (built by ``python -m exact_attention_05_amd.build``)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_05_amd.build`")
        L = ctypes.CDLL(path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_forward.restype = i
        L.fa_backward_workspace_size.argtypes = [i, i, i, i, i, i]
        L.fa_backward_workspace_size.restype = sz
        L.fa_backward_gqa_workspace_size.argtypes = [i, i, i, i, i, i, i]
        L.fa_backward_gqa_workspace_size.restype = sz
        L.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                  i, i, i, i, i, f, i, i, vp]
        L.fa_backward.restype = i
        L.fa_backward_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, vp]
        L.fa_backward_preprocess.restype = i
        L.fa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_backward_dkdv.restype = i
        L.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_backward_dq.restype = i
        L.fa_forward_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.fa_forward_gqa.restype = i
        L.fa_backward_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                      i, i, i, i, i, i, f, i, i, vp]
        L.fa_backward_gqa.restype = i
        L.fa_forward_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, i, vp]
        L.fa_forward_ext.restype = i
        L.fa_backward_ext.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                      i, i, i, i, i, i, f, i, i, i, i, vp]
        L.fa_backward_ext.restype = i
        L.fa_forward_merge.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, f, i, i, i, i, vp]
        L.fa_forward_merge.restype = i
        L.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_backward_noalloc.restype = i
        ll = ctypes.c_longlong
        L.fa_lse_merge.argtypes = [vp, vp, vp, vp, i, ll, i, i, i, vp]
        L.fa_lse_merge.restype = i
        L.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, i, i, i, vp]
        L.fa_decode.restype = i
        L.fa_decode_workspace_size.argtypes = [i, i, i, i, i]
        L.fa_decode_workspace_size.restype = sz
        L.fa_decode_splits.argtypes = [i, i, i, i, i]
        L.fa_decode_splits.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        L.fa_version.restype = i
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def version() -> int:
    return int(lib().fa_version())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be (B, H, n, d), got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype not in _DTYPES:
            raise ValueError(f"{name}: dtype {t.dtype} not supported (float32 or bfloat16)")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, n_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    h_kv = k.shape[1]
    if h_kv < 1 or H % h_kv != 0:
        raise ValueError(f"k and v have {h_kv} heads, which must divide q's {H}")
    return B, H, n_q, k.shape[2], d


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            q_offset: int = 0, window: int | None = None):
    """O, LSE = attention(q, k, v).  q: (B,H,n_q,d); k, v: (B,H_kv,n_k,d) with H_kv
    dividing H (H_kv < H shares each K/V head among H/H_kv consecutive query
    heads: grouped-query or, with H_kv = 1, multi-query attention).

    Returns O (q's dtype, (B,H,n_q,d)) and LSE (float32, (B,H,n_q)).
    ``scale`` defaults to 1/sqrt(d).  ``q_offset`` places query row i at key
    position i + q_offset for the causal mask and the window; ``window`` = w
    keeps only keys within +-w of that position (None: no window).  A row that
    sees no key gets O = 0 and LSE = -inf.
    """
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 (B, H, n_q) tensor")
    h_kv = k.shape[1]
    if q_offset != 0 or window is not None:
        st = lib().fa_forward_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, h_kv, n_q,
                                  n_k, d, _scale(scale, d), int(bool(causal)), int(q_offset),
                                  -1 if window is None else int(window), _DTYPES[q.dtype],
                                  _stream(q.device))
        _check(st, "fa_forward_ext")
    elif h_kv == H:
        st = lib().fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, n_q, n_k, d,
                              _scale(scale, d), int(bool(causal)), _DTYPES[q.dtype], _stream(q.device))
        _check(st, "fa_forward")
    else:
        st = lib().fa_forward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, h_kv, n_q,
                                  n_k, d, _scale(scale, d), int(bool(causal)), _DTYPES[q.dtype],
                                  _stream(q.device))
        _check(st, "fa_forward_gqa")
    return out, lse


def forward_merge(q, k, v, o_prior, lse_prior, causal: bool = False, scale: float | None = None,
                  q_offset: int = 0, window: int | None = None, out=None, lse=None,
                  out_dtype: torch.dtype | None = None):
    """Attention of q over this call's k, v merged into a prior result over
    other keys (fa_forward_merge): returns (o, lse) over both key sets.

    o_prior (B,H,n_q,d) float32 or q's dtype and lse_prior (B,H,n_q) float32
    hold the result so far (lse_prior = -inf: no prior for that row).  ``out``
    and ``lse`` may be o_prior and lse_prior themselves (in-place
    accumulation); otherwise they are allocated with ``out_dtype`` (default
    o_prior's dtype).  Masks as forward()."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    if o_prior.shape != q.shape or o_prior.dtype not in (torch.float32, q.dtype) or \
            not o_prior.is_contiguous() or o_prior.device != q.device:
        raise ValueError("o_prior must be a contiguous (B, H, n_q, d) float32 or q-dtype tensor on q's device")
    if lse_prior.shape != (B, H, n_q) or lse_prior.dtype != torch.float32 or not lse_prior.is_contiguous():
        raise ValueError("lse_prior must be a contiguous float32 (B, H, n_q) tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=o_prior.dtype if out_dtype is None else out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype not in (torch.float32, q.dtype) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, H, n_q, d) float32 or q-dtype tensor")
    if lse.shape != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, n_q) tensor")
    st = lib().fa_forward_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(o_prior), _ptr(lse_prior),
                                _DTYPES[o_prior.dtype], _ptr(out), _ptr(lse), _DTYPES[out.dtype],
                                B, H, k.shape[1], n_q, n_k, d, _scale(scale, d), int(bool(causal)),
                                int(q_offset), -1 if window is None else int(window), _DTYPES[q.dtype],
                                _stream(q.device))
    _check(st, "fa_forward_merge")
    return out, lse


def backward_workspace_size(B, H, n_q, n_k, d, dtype: torch.dtype, H_kv: int | None = None) -> int:
    """Workspace bytes of the backward pass (with H_kv K/V heads shared by the
    H query heads: the size fa_backward_gqa / fa_backward_ext need)."""
    if H_kv is None or H_kv == H:
        return int(lib().fa_backward_workspace_size(B, H, n_q, n_k, d, _DTYPES[dtype]))
    return int(lib().fa_backward_gqa_workspace_size(B, H, H_kv, n_q, n_k, d, _DTYPES[dtype]))


def _check_like(name, t, ref):
    if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() or t.device != ref.device:
        raise ValueError(f"{name} must be a contiguous tensor shaped and typed like {tuple(ref.shape)} {ref.dtype}")


def backward(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, q_offset: int = 0,
             window: int | None = None):
    """dQ, dK, dV from the saved o and lse of ``forward``; dK, dV have k's shape."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    _check_like("o", o, q)
    _check_like("do", do, q)
    if lse.shape != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, n_q) tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_like("dq", dq, q)
    _check_like("dk", dk, k)
    _check_like("dv", dv, v)
    h_kv = k.shape[1]
    if workspace is None:
        workspace = backward_workspace(B, H, n_q, n_k, d, q.dtype, q.device, H_kv=h_kv)
    if q_offset != 0 or window is not None:
        st = lib().fa_backward_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), *_ws(workspace),
                                   B, H, h_kv, n_q, n_k, d, _scale(scale, d), int(bool(causal)),
                                   int(q_offset), -1 if window is None else int(window),
                                   _DTYPES[q.dtype], _stream(q.device))
        _check(st, "fa_backward_ext")
    elif h_kv == H:
        st = lib().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), *_ws(workspace),
                               B, H, n_q, n_k, d, _scale(scale, d), int(bool(causal)),
                               _DTYPES[q.dtype], _stream(q.device))
        _check(st, "fa_backward")
    else:
        st = lib().fa_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), *_ws(workspace),
                                   B, H, h_kv, n_q, n_k, d, _scale(scale, d), int(bool(causal)),
                                   _DTYPES[q.dtype], _stream(q.device))
        _check(st, "fa_backward_gqa")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal: bool = False, scale: float | None = None):
    """fa_backward_noalloc: the backward pass into the caller's dq, dk, dv
    with the library's fixed device scratch as the workspace (no device
    allocation by the library or here).  One K/V head per query head."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    _require_mha(q, k, "backward_noalloc")
    for name, t, ref in (("o", o, q), ("do", do, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_like(name, t, ref)
    if lse.shape != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, n_q) tensor")
    st = lib().fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                   _ptr(dk), _ptr(dv), B, H, n_q, n_k, d, _scale(scale, d),
                                   int(bool(causal)), _DTYPES[q.dtype], _stream(q.device))
    _check(st, "fa_backward_noalloc")
    return dq, dk, dv


def backward_workspace(B, H, n_q, n_k, d, dtype: torch.dtype, device, H_kv: int | None = None) -> torch.Tensor:
    """A device buffer of backward_workspace_size bytes (256-byte aligned)."""
    n = backward_workspace_size(B, H, n_q, n_k, d, dtype, H_kv)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws(workspace):
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def workspace_delta(workspace: torch.Tensor, B: int, H: int, n_q: int) -> torch.Tensor:
    """View of the row sums D = rowsum(dO * O) that stage 1 writes at the start
    of the workspace, as a float32 (B, H, n_q) tensor."""
    return workspace[: B * H * n_q * 4].view(torch.float32).view(B, H, n_q)


def backward_preprocess(o, do, lse, workspace=None):
    """Stage 1: writes D = rowsum(do * o) and LSE * log2(e) into the workspace
    (allocated if not given) and returns it."""
    B, H, n_q, d = o.shape
    _check_like("do", do, o)
    if workspace is None:
        workspace = backward_workspace(B, H, n_q, n_q, d, o.dtype, o.device)
    st = lib().fa_backward_preprocess(_ptr(o), _ptr(do), _ptr(lse), *_ws(workspace), B, H, n_q, d,
                                      _DTYPES[o.dtype], _stream(o.device))
    _check(st, "fa_backward_preprocess")
    return workspace


def _require_mha(q, k, where):
    if k.shape[1] != q.shape[1]:
        raise ValueError(f"{where}: the stage entry points take one K/V head per query head; "
                         "use backward() for shared K/V heads")


def backward_dkdv(q, k, v, do, workspace, causal=False, scale=None, dk=None, dv=None):
    """Stage 2: dK and dV from the workspace of stage 1."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    _require_mha(q, k, "backward_dkdv")
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = lib().fa_backward_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), *_ws(workspace),
                                _ptr(dk), _ptr(dv), B, H, n_q, n_k, d, _scale(scale, d),
                                int(bool(causal)), _DTYPES[q.dtype], _stream(q.device))
    _check(st, "fa_backward_dkdv")
    return dk, dv


def backward_dq(q, k, v, do, workspace, causal=False, scale=None, dq=None):
    """Stage 3: dQ from the workspace of stage 1."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    _require_mha(q, k, "backward_dq")
    dq = torch.empty_like(q) if dq is None else dq
    st = lib().fa_backward_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), *_ws(workspace), _ptr(dq),
                              B, H, n_q, n_k, d, _scale(scale, d), int(bool(causal)),
                              _DTYPES[q.dtype], _stream(q.device))
    _check(st, "fa_backward_dq")
    return dq


def lse_merge(o_parts, lse_parts, out_dtype: torch.dtype | None = None, out=None, lse=None):
    """Merge attention results over disjoint key sets (fa_lse_merge).

    o_parts: (P, ..., d) float32 or bfloat16, lse_parts: (P, ...) float32,
    both contiguous on the GPU.  Returns (o, lse) of shapes (..., d), (...):
    lse = ln sum_p exp(lse_p), o = sum_p exp(lse_p - lse) o_p.  ``out_dtype``
    defaults to the parts' dtype."""
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if o_parts.dtype not in _DTYPES or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts must be float32 or bfloat16 and lse_parts float32")
    if o_parts.dim() < 2 or tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape):
        raise ValueError(f"o_parts {tuple(o_parts.shape)} and lse_parts {tuple(lse_parts.shape)} do not match")
    n_parts, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    out_dtype = o_parts.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise ValueError(f"out_dtype {out_dtype} not supported")
    shape = tuple(o_parts.shape[1:])
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty(shape[:-1], dtype=torch.float32, device=o_parts.device)
    if tuple(out.shape) != shape or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the merged shape and out_dtype")
    if tuple(lse.shape) != shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of the merged row shape")
    st = lib().fa_lse_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse), n_parts, rows, d,
                            _DTYPES[o_parts.dtype], _DTYPES[out_dtype], _stream(o_parts.device))
    _check(st, "fa_lse_merge")
    return out, lse


def decode_splits(B, H, H_kv, n_q, n_k) -> int:
    """The library's default number of key chunks for fa_decode."""
    return int(lib().fa_decode_splits(B, H, H_kv, n_q, n_k))


def decode_workspace_size(B, H, n_q, d, n_splits) -> int:
    return int(lib().fa_decode_workspace_size(B, H, n_q, d, n_splits))


def decode(q, k, v, causal: bool = True, scale: float | None = None, q_offset: int | None = None,
           window: int | None = None, n_splits: int | None = None, out=None, lse=None,
           workspace=None):
    """Split-KV decoding (fa_decode, bfloat16): a few query rows q (B,H,n_q,d)
    against a long K/V cache k, v (B,H_kv,n_k,d).  ``q_offset`` defaults to
    n_k - n_q (the queries are the last n_q positions); masks as forward().
    ``n_splits`` defaults to decode_splits(); the workspace is allocated when
    not given.  Returns (o, lse)."""
    B, H, n_q, n_k, d = _check_qkv(q, k, v)
    h_kv = k.shape[1]
    off = n_k - n_q if q_offset is None else int(q_offset)
    splits = decode_splits(B, H, h_kv, n_q, n_k) if n_splits is None else int(n_splits)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check_like("out", out, q)
    if lse.shape != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, n_q) tensor")
    if workspace is None:
        n = decode_workspace_size(B, H, n_q, d, max(1, splits))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    st = lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *_ws(workspace),
                         B, H, h_kv, n_q, n_k, d, _scale(scale, d), int(bool(causal)), off,
                         -1 if window is None else int(window), splits, _DTYPES[q.dtype],
                         _stream(q.device))
    _check(st, "fa_decode")
    return out, lse

