"""Host-side checks of the C ABI: the library loads, exports every function
include/fa.h declares, and rejects invalid arguments before launching
anything.  Each call here fails validation on the host, so no GPU is needed
and no kernel runs."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_05_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake, suitably aligned device addresses: never dereferenced, because every
# call below fails validation first.
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100008)  # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"fa_forward", "fa_backward", "fa_backward_workspace_size", "fa_status_string"} <= set(names)
    L = fa.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (fa_[a-z_]+)\b", out.stdout))
    assert set(names) <= exported


def test_status_strings_cover_every_code():
    seen = set()
    for code in range(7):
        s = fa.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert fa.status_string(99) == "unknown status"
    assert fa.status_string(-1) == "unknown status"


def test_version():
    assert fa.version() >= 10000


def fwd(q=P, k=P, v=P, o=P2, lse=P2, B=1, H=1, n_q=8, n_k=8, d=64, scale=0.125, causal=0, dtype=1):
    return fa.lib().fa_forward(q, k, v, o, lse, B, H, n_q, n_k, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, fa.FA_ERR_INVALID_ARG),
    ({"k": None}, fa.FA_ERR_INVALID_ARG),
    ({"v": None}, fa.FA_ERR_INVALID_ARG),
    ({"o": None}, fa.FA_ERR_INVALID_ARG),
    ({"lse": None}, fa.FA_ERR_INVALID_ARG),
    ({"B": 0}, fa.FA_ERR_INVALID_ARG),
    ({"H": -1}, fa.FA_ERR_INVALID_ARG),
    ({"n_q": 0}, fa.FA_ERR_INVALID_ARG),
    ({"n_k": 0}, fa.FA_ERR_INVALID_ARG),
    ({"d": 48}, fa.FA_ERR_UNSUPPORTED),
    ({"d": 256}, fa.FA_ERR_UNSUPPORTED),
    ({"dtype": 7}, fa.FA_ERR_UNSUPPORTED),
    ({"causal": 2}, fa.FA_ERR_INVALID_ARG),
    ({"scale": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"scale": float("inf")}, fa.FA_ERR_INVALID_ARG),
    ({"scale": -0.5}, fa.FA_ERR_INVALID_ARG),
    ({"q": MIS}, fa.FA_ERR_ALIGNMENT),
    ({"o": MIS}, fa.FA_ERR_ALIGNMENT),
    ({"lse": ctypes.c_void_p(0x100002)}, fa.FA_ERR_ALIGNMENT),
    ({"B": 65536, "H": 65536}, fa.FA_ERR_INVALID_ARG),
    ({"B": 1 << 20, "H": 64, "n_q": 1 << 20}, fa.FA_ERR_INVALID_ARG),
])
def test_forward_rejects_invalid_arguments(kw, code):
    assert fwd(**kw) == code


def test_workspace_size():
    L = fa.lib()
    # two float32 row vectors, each with >= 16 bytes of slack, 256-byte multiples
    assert L.fa_backward_workspace_size(2, 16, 4096, 4096, 128, 1) == 2 * (2 * 16 * 4096 * 4 + 256)
    assert L.fa_backward_workspace_size(1, 1, 3, 3, 64, 0) == 512
    assert L.fa_backward_workspace_size(1, 1, 60, 3, 64, 0) == 512
    assert L.fa_backward_workspace_size(1, 1, 61, 3, 64, 0) == 1024
    assert L.fa_backward_workspace_size(1, 1, 0, 3, 64, 0) == 0
    assert L.fa_backward_workspace_size(1, 1, 3, 3, 40, 0) == 0


def bwd(ws=P2, ws_bytes=1 << 20, B=1, H=1, n_q=8, n_k=8, d=64, scale=0.125, causal=0, dtype=1,
        dq=P2, o=P):
    return fa.lib().fa_backward(P, P, P, o, P, P, dq, P2, P2, ws, ws_bytes, B, H, n_q, n_k, d,
                                scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    ({"ws": None}, fa.FA_ERR_WORKSPACE),
    ({"ws_bytes": 511}, fa.FA_ERR_WORKSPACE),
    ({"ws": ctypes.c_void_p(0x100010)}, fa.FA_ERR_ALIGNMENT),
    ({"dq": None}, fa.FA_ERR_INVALID_ARG),
    ({"o": MIS}, fa.FA_ERR_ALIGNMENT),
    ({"d": 96}, fa.FA_ERR_UNSUPPORTED),
    ({"causal": -1}, fa.FA_ERR_INVALID_ARG),
    ({"n_k": 0}, fa.FA_ERR_INVALID_ARG),
])
def test_backward_rejects_invalid_arguments(kw, code):
    assert bwd(**kw) == code


def test_stage_entry_points_reject_invalid_arguments():
    L = fa.lib()
    W = 1 << 20
    assert L.fa_backward_preprocess(P, None, P2, P2, W, 1, 1, 8, 64, 1, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_preprocess(P, P, P2, P2, W, 1, 1, 8, 40, 1, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_backward_preprocess(P, P, P2, P2, 100, 1, 1, 8, 64, 1, None) == fa.FA_ERR_WORKSPACE
    assert L.fa_backward_preprocess(P, P, P2, ctypes.c_void_p(0x200080), W, 1, 1, 8, 64, 1, None) == fa.FA_ERR_ALIGNMENT
    assert L.fa_backward_dkdv(P, P, P, P, P2, W, None, P2, 1, 1, 8, 8, 64, 0.1, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_dkdv(P, P, P, P, P2, W, P2, P2, 1, 1, 8, 8, 64, -0.1, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_dkdv(P, P, P, P, None, W, P2, P2, 1, 1, 8, 8, 64, 0.1, 0, 1, None) == fa.FA_ERR_WORKSPACE
    assert L.fa_backward_dq(P, P, P, P, P2, W, MIS, 1, 1, 8, 8, 64, 0.1, 0, 1, None) == fa.FA_ERR_ALIGNMENT
    assert L.fa_backward_dq(P, P, P, P, P2, W, P2, 1, 0, 8, 8, 64, 0.1, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_dq(P, P, P, P, P2, 0, P2, 1, 1, 8, 8, 64, 0.1, 0, 1, None) == fa.FA_ERR_WORKSPACE


def test_binding_validates_shapes_before_calling():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)  # CPU tensors are refused before any library call


@pytest.mark.parametrize("H,H_kv", [(8, 0), (8, 3), (8, 16), (4, -1)])
def test_gqa_rejects_bad_head_counts(H, H_kv):
    L = fa.lib()
    assert L.fa_forward_gqa(P, P, P, P2, P2, 1, H, H_kv, 8, 8, 64, 0.125, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_gqa(P, P, P, P, P, P, P2, P2, P2, P2, 1 << 20, 1, H, H_kv, 8, 8, 64, 0.125,
                             0, 1, None) == fa.FA_ERR_INVALID_ARG


def test_gqa_validates_like_forward():
    L = fa.lib()
    assert L.fa_forward_gqa(P, P, P, P2, P2, 1, 8, 2, 8, 8, 48, 0.125, 0, 1, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_forward_gqa(P, MIS, P, P2, P2, 1, 8, 2, 8, 8, 64, 0.125, 0, 1, None) == fa.FA_ERR_ALIGNMENT
    assert L.fa_backward_gqa(P, P, P, P, P, P, P2, P2, P2, None, 1 << 20, 1, 8, 2, 8, 8, 64, 0.125,
                             0, 1, None) == fa.FA_ERR_WORKSPACE


@pytest.mark.parametrize("n,q_offset,window", [(8, (1 << 29) + 1, -1), (8, -(1 << 29) - 1, -1),
                                                (8, 0, -2), (8, 0, (1 << 29) + 1),
                                                ((1 << 29) + 1, 0, 5), ((1 << 29) + 1, 3, -1)])
def test_ext_rejects_out_of_range_band(n, q_offset, window):
    L = fa.lib()
    assert L.fa_forward_ext(P, P, P, P2, P2, 1, 2, 2, n, 8, 64, 0.125, 1, q_offset, window, 1,
                            None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_backward_ext(P, P, P, P, P, P, P2, P2, P2, P2, 1 << 20, 1, 2, 2, 8, n, 64, 0.125, 1,
                             q_offset, window, 1, None) == fa.FA_ERR_INVALID_ARG



# ---------------------------------------------------- decoding and merging

def dec(q=P, k=P, v=P, o=P2, lse=P2, ws=None, ws_bytes=0, B=1, H=8, H_kv=2, n_q=1, n_k=4096, d=128,
        scale=0.088, causal=1, q_offset=4095, window=-1, n_splits=4, dtype=1):
    return fa.lib().fa_decode(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, n_q, n_k, d, scale, causal,
                              q_offset, window, n_splits, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(n_splits=65537), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED),           # float32 decoding is not provided
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(window=-2), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=MIS), fa.FA_ERR_ALIGNMENT),
    (dict(), fa.FA_ERR_WORKSPACE),                      # 4 chunks, no workspace
    (dict(ws=P, ws_bytes=1024), fa.FA_ERR_WORKSPACE),   # too small
    (dict(ws=ctypes.c_void_p(0x100010), ws_bytes=1 << 30), fa.FA_ERR_ALIGNMENT),
])
def test_decode_rejects(kw, code):
    assert dec(**kw) == code


def test_decode_workspace_size():
    # float32 partial outputs and LSE per chunk, each rounded up to 256 bytes
    assert fa.decode_workspace_size(1, 8, 1, 128, 1) == 0
    rows = 2 * 8 * 3
    expect = -(-4 * rows * 128 * 4 // 256) * 256 + -(-4 * rows * 4 // 256) * 256
    assert fa.decode_workspace_size(2, 8, 3, 128, 4) == expect
    assert fa.decode_workspace_size(2, 8, 3, 96, 4) == 0
    assert fa.decode_workspace_size(0, 8, 3, 128, 4) == 0


def test_decode_splits():
    # enough (batch, K/V head, row block, chunk) workgroups for one per
    # compute unit, chunks of at least 256 keys
    assert fa.decode_splits(4, 64, 8, 1, 32768) == 8      # 32 units -> 8 chunks of 4096 keys
    assert fa.decode_splits(1, 8, 8, 1, 1000) == 3        # at most n_k / 256
    assert fa.decode_splits(64, 32, 32, 1, 4096) == 1     # 2048 units already
    assert fa.decode_splits(1, 8, 3, 1, 4096) == 0        # H_kv must divide H


def merge(op=P, lp=P2, o=P, lse=P2, n_parts=2, rows=16, d=64, pdt=0, odt=1):
    return fa.lib().fa_lse_merge(op, lp, o, lse, n_parts, rows, d, pdt, odt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_parts=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(pdt=2), fa.FA_ERR_UNSUPPORTED),
    (dict(odt=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(op=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=MIS), fa.FA_ERR_ALIGNMENT),
    (dict(lse=ctypes.c_void_p(0x200002)), fa.FA_ERR_ALIGNMENT),
    (dict(rows=1 << 40), fa.FA_ERR_INVALID_ARG),
])
def test_lse_merge_rejects(kw, code):
    assert merge(**kw) == code


def test_gqa_backward_workspace_size():
    L = fa.lib()
    base = L.fa_backward_workspace_size(1, 32, 4096, 4096, 128, 1)
    # one run per K/V head when there is no sharing
    assert L.fa_backward_gqa_workspace_size(1, 32, 32, 4096, 4096, 128, 1) == base
    # one K/V head: each of the 32 query heads is a run of its own, and each
    # run's float32 partial dK and dV are kept
    part = 32 * 1 * 4096 * 128 * 4
    assert L.fa_backward_gqa_workspace_size(1, 32, 1, 4096, 4096, 128, 1) == base + 2 * part
    # 8 K/V heads, 4 query heads each: 4 runs per K/V head
    part8 = 4 * 8 * 4096 * 128 * 4
    assert L.fa_backward_gqa_workspace_size(1, 32, 8, 4096, 4096, 128, 0) == base + 2 * part8
    assert L.fa_backward_gqa_workspace_size(1, 32, 3, 64, 64, 64, 1) == 0


def test_gqa_backward_rejects_a_workspace_without_room_for_the_runs():
    L = fa.lib()
    base = L.fa_backward_workspace_size(1, 8, 256, 256, 64, 1)
    st = L.fa_backward_gqa(P, P, P, P, P, P2, P2, P2, P2, ctypes.c_void_p(0x400000), base,
                           1, 8, 2, 256, 256, 64, 0.125, 0, 1, None)
    assert st == fa.FA_ERR_WORKSPACE


def test_gqa_runs_grow_when_the_partials_would_pass_4_gib():
    L = fa.lib()
    # 64 query heads on one K/V head at n_k = 131072: one-head runs would need
    # 2 * 64 * 131072 * 128 * 4 B = 8 GiB; runs of two heads need 4 GiB
    base = L.fa_backward_workspace_size(1, 64, 16, 131072, 128, 1)
    got = L.fa_backward_gqa_workspace_size(1, 64, 1, 16, 131072, 128, 1)
    assert got == base + 2 * 32 * 131072 * 128 * 4



def fmerge(q=P, k=P, v=P, op=ctypes.c_void_p(0x300000), lp=ctypes.c_void_p(0x380000), pdt=1,
           o=ctypes.c_void_p(0x400000), lse=ctypes.c_void_p(0x480000), odt=1, B=1, H=2, H_kv=2,
           n_q=8, n_k=8, d=64, scale=0.125, causal=0, q_offset=0, window=-1, dtype=1):
    return fa.lib().fa_forward_merge(q, k, v, op, lp, pdt, o, lse, odt, B, H, H_kv, n_q, n_k, d, scale,
                                     causal, q_offset, window, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), fa.FA_ERR_INVALID_ARG),
    (dict(lp=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(op=MIS), fa.FA_ERR_ALIGNMENT),
    (dict(lp=ctypes.c_void_p(0x380002)), fa.FA_ERR_ALIGNMENT),
    (dict(pdt=2), fa.FA_ERR_UNSUPPORTED),
    (dict(odt=5), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0, pdt=1, odt=0), fa.FA_ERR_UNSUPPORTED),   # float32 inputs keep a float32 result
    (dict(dtype=0, pdt=0, odt=1), fa.FA_ERR_UNSUPPORTED),
    (dict(o=ctypes.c_void_p(0x300000), odt=0), fa.FA_ERR_INVALID_ARG),  # in place, dtypes differ
    (dict(o=ctypes.c_void_p(0x300010)), fa.FA_ERR_INVALID_ARG),         # partial overlap of o and o_prior
    (dict(lse=ctypes.c_void_p(0x380004)), fa.FA_ERR_INVALID_ARG),       # partial overlap of the LSE rows
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(window=-2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
])
def test_forward_merge_rejects(kw, code):
    assert fmerge(**kw) == code


def test_backward_noalloc_rejects_before_touching_the_gpu():
    # Sizes whose workspace would pass the fixed 16 MiB scratch are refused
    # with their own status, as are invalid arguments, all on the host.
    L = fa.lib()

    def call(B=1, H=2, n_q=8, n_k=8, d=64, dq=P2, causal=0):
        return L.fa_backward_noalloc(P, P, P, P, P, P2, dq, P2, P2, B, H, n_q, n_k, d, 0.125, causal, 1, None)

    assert call(B=1, H=32, n_q=65536) == fa.FA_ERR_TOO_LARGE   # 2 x 8 MiB + slack
    assert call(B=64, H=64, n_q=4096) == fa.FA_ERR_TOO_LARGE
    assert call(dq=None) == fa.FA_ERR_INVALID_ARG
    assert call(d=80) == fa.FA_ERR_UNSUPPORTED
    assert call(causal=3) == fa.FA_ERR_INVALID_ARG
    assert call(dq=MIS) == fa.FA_ERR_ALIGNMENT
