"""Exact scaled dot-product attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI declared in
``include/fa.h`` (library ``lib/libfa.so``); this package is its Python
binding.  See ``forward`` and ``backward``; ``decode`` (split-KV decoding
against a long K/V cache) and ``lse_merge`` (attention results over disjoint
key sets combined into the result over all keys) and ``forward_merge`` (a
forward pass that merges into a prior result in its epilogue).
"""
from .binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_FP32,
    FA_ERR_ALIGNMENT,
    FA_ERR_INVALID_ARG,
    FA_ERR_LAUNCH,
    FA_ERR_TOO_LARGE,
    FA_ERR_UNSUPPORTED,
    FA_ERR_WORKSPACE,
    FA_OK,
    FaError,
    backward,
    backward_noalloc,
    backward_dkdv,
    backward_dq,
    backward_preprocess,
    backward_workspace,
    backward_workspace_size,
    decode,
    decode_splits,
    decode_workspace_size,
    forward,
    forward_merge,
    lse_merge,
    lib,
    library_path,
    status_string,
    version,
    workspace_delta,
)
