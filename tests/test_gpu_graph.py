"""GPU check that the library's launches can be recorded into a HIP graph
and replayed.  A training or serving loop that replays a captured step needs
the entry points to issue nothing but kernel launches on the caller's stream:
no allocation, no memset, no synchronisation.  The forward pass, the three
backward stages and the non-allocating backward are captured with
preallocated outputs and workspace, replayed several times with eager work
and synchronisations between the replays, and every replay must equal the
eager calls bit for bit; between replays the inputs are overwritten in place,
so each replay must read the live buffers, and the outputs are poisoned, so
each replay must write all of them."""
import pytest
import torch

import exact_attention_05_amd as fa
import workloads
from parity import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


CASES = [  # B, H, n_q, n_k, d, causal, dtype
    (1, 8, 1000, 1000, 128, False, torch.bfloat16),
    (2, 4, 777, 777, 128, True, torch.bfloat16),
    (1, 4, 300, 520, 64, False, torch.float32),
]


def _draw(seed, case, dev):
    B, H, n_q, n_k, d, causal, dtype = case
    return [t.to(dev) for t in workloads.random_qkv(seed, B, H, n_q, n_k, d, dtype, with_do=True)]


def _eager(q, k, v, do, causal):
    o, lse = fa.forward(q, k, v, causal=causal)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    return [o, lse, dq, dk, dv]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}nq{}nk{}d{}c{:d}{}".format(
    *c[:6], "bf16" if c[6] == torch.bfloat16 else "fp32"))
def test_forward_backward_replay_from_a_graph(dev, case):
    B, H, n_q, n_k, d, causal, dtype = case
    q, k, v, do = _draw(7100, case, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = fa.backward_workspace(B, H, n_q, n_k, d, dtype, dev)
    outs = [o, lse, dq, dk, dv]

    # one eager pass first: the library's one-time device queries happen here
    _eager(q, k, v, do, causal)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward(q, k, v, causal=causal, out=o, lse=lse)
        fa.backward_preprocess(o, do, lse, workspace=ws)
        fa.backward_dkdv(q, k, v, do, ws, causal=causal, dk=dk, dv=dv)
        fa.backward_dq(q, k, v, do, ws, causal=causal, dq=dq)

    for rep in range(3):
        new = _draw(7101 + rep, case, dev)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = _eager(*new, causal)  # eager calls on the same inputs, between replays
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_noalloc_backward_replays_from_a_graph(dev):
    # The backward for callers that cannot allocate, as such a caller would
    # use it: recorded into a graph.  Its first call on the device (the
    # scratch lookup) happens before the capture.
    case = (1, 8, 900, 900, 128, True, torch.bfloat16)
    B, H, n_q, n_k, d, causal, dtype = case
    q, k, v, do = _draw(7200, case, dev)
    o, lse = fa.forward(q, k, v, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal=causal)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal=causal)
    for rep in range(3):
        new = _draw(7201 + rep, case, dev)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        o2, lse2 = fa.forward(q, k, v, causal=causal)
        o.copy_(o2)
        lse.copy_(lse2)
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dq, dk, dv)]
        ref = fa.backward(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from fa_backward"
