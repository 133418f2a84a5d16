"""GPU check of fa_backward_noalloc, the backward pass for callers that
cannot allocate device memory: its workspace is the library's fixed device
scratch.  Its results must equal fa_backward's bit for bit (the same kernels
on the same inputs), on two calls in a row, the second smaller, so that the
second call cannot rely on anything the first left behind; and the calls
must not allocate device memory.  The first call on a device is its set-up:
the library looks up the scratch's address there, and the HIP runtime maps
the 16 MiB array on that device then; after it, free device memory does not
move."""
import pytest
import torch

import exact_attention_05_amd as fa
import workloads
from parity import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


CALLS = [  # B, H, n_q, n_k, d, causal, dtype: the second call of each pair is smaller
    [(2, 16, 1000, 1000, 128, True, torch.bfloat16), (1, 3, 257, 300, 64, False, torch.bfloat16)],
    [(1, 8, 600, 555, 64, False, torch.float32), (1, 2, 17, 17, 32, True, torch.float32)],
]


def _setup_call(dev):
    q, k, v, do = (t.to(dev) for t in workloads.random_qkv(6999, 1, 1, 8, 8, 32, torch.bfloat16, with_do=True))
    o, lse = fa.forward(q, k, v)
    fa.backward_noalloc(q, k, v, o, do, lse, torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    torch.cuda.synchronize()


@pytest.mark.parametrize("pair", CALLS, ids=["bf16", "fp32"])
def test_noalloc_backward_equals_backward(dev, pair):
    _setup_call(dev)
    for i, (B, H, n_q, n_k, d, causal, dtype) in enumerate(pair):
        q, k, v, do = (t.to(dev) for t in workloads.random_qkv(7000 + 13 * i + d, B, H, n_q, n_k, d, dtype,
                                                                with_do=True))
        o, lse = fa.forward(q, k, v, causal=causal)
        ref = fa.backward(q, k, v, o, do, lse, causal=causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        fa.backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal=causal)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert free0 == free1, f"the call changed free device memory by {free0 - free1} bytes"
        for name, a, b in zip(("dQ", "dK", "dV"), ref, (dq, dk, dv)):
            assert torch.equal(a, b), f"call {i} {(B, H, n_q, n_k, d, causal, dtype)}: {name} differs"


def test_noalloc_refuses_sizes_beyond_its_scratch(dev):
    B, H, n, d = 1, 32, 65536, 32   # workspace 2 x 8 MiB + slack: past the 16 MiB scratch
    q = torch.zeros(B, H, n, d, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, n, dtype=torch.float32, device=dev)
    with pytest.raises(fa.FaError) as e:
        fa.backward_noalloc(q, q, q, q, q, lse, q.clone(), q.clone(), q.clone())
    assert e.value.status == fa.FA_ERR_TOO_LARGE
