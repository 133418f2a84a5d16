"""GPU parity of the forward pass against the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import exact_attention_05_amd as fa
import oracle
import workloads
from parity import TOL_LSE, assert_close, fp32_score_tol, np64, require_gpu, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def run_fwd(dev, q, k, v, scale, causal):
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_full(dev, q, k, v, scale, causal, tag="", tol=None):
    o, lse = run_fwd(dev, q, k, v, scale, causal)
    ro, rl = oracle.attention_fwd(np64(q), np64(k), np64(v), scale, causal)
    assert_close(f"O {tag}", o, ro, tol_for(q.dtype) if tol is None else tol)
    assert_close(f"LSE {tag}", lse, rl, TOL_LSE)
    return o, lse


# ----------------------------------------------------------- the workloads

def test_c1_fp32_b2_h3_n128_d32(dev):
    w = workloads.c1()
    check_full(dev, w.q, w.k, w.v, w.scale, w.causal, w.name)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_c2_single_head_n4096_d64(dev, dtype):
    w = workloads.c2(dtype)
    o, lse = check_full(dev, w.q, w.k, w.v, w.scale, False, w.name)
    # Query rows are independent: 128-row slices give bitwise the full result.
    for start in (0, 128, 1920, 3968):
        os_, ls_ = run_fwd(dev, w.q[:, :, start:start + 128].contiguous(), w.k, w.v, w.scale, False)
        assert torch.equal(os_, o[:, :, start:start + 128])
        assert torch.equal(ls_, lse[:, :, start:start + 128])


@pytest.mark.parametrize("causal", [False, True])
def test_c3_b1_h32_n4096_d128(dev, causal):
    # Every head, element by element against the full fp64 oracle (its
    # 4096 x 4096 score matrix materialised per head).
    w = workloads.c3(causal)
    o, lse = run_fwd(dev, w.q, w.k, w.v, w.scale, causal)
    worst_o = worst_l = 0.0
    for h in range(w.q.shape[1]):
        fo, fl = oracle.attention_fwd(np64(w.q[0, h]), np64(w.k[0, h]), np64(w.v[0, h]), w.scale, causal)
        worst_o = max(worst_o, assert_close(f"O {w.name} head {h}", o[0, h], fo, tol_for(w.q.dtype)))
        worst_l = max(worst_l, assert_close(f"LSE {w.name} head {h}", lse[0, h], fl, TOL_LSE))
    print(f"{w.name}: all 32 heads, max |err| O {worst_o:.3e}, LSE {worst_l:.3e}")


def test_c4_long_context_causal_n16384(dev):
    w = workloads.c4()
    o, lse = run_fwd(dev, w.q, w.k, w.v, w.scale, True)
    rows = workloads.c4_rows(256)
    ro, rl = oracle.attention_rows(w.q.float().numpy(), w.k.float().numpy(), w.v.float().numpy(),
                                   rows, w.scale, True)
    got_o = np.stack([np64(o[b, h, i]) for b, h, i in rows])
    got_l = np.array([float(lse[b, h, i]) for b, h, i in rows])
    assert_close("O rows c4", got_o, ro, tol_for(w.q.dtype), rounded_bf16=True)
    assert_close("LSE rows c4", got_l, rl, TOL_LSE)


# --------------------------------------------------- shapes and edge cases

SHAPES = [
    (1, 1, 1, 1), (1, 2, 17, 17), (2, 1, 63, 65), (1, 1, 65, 63), (1, 3, 129, 129),
    (1, 1, 257, 300), (1, 1, 300, 257), (1, 2, 1000, 1000), (1, 1, 5, 700), (1, 1, 700, 5),
]


@pytest.mark.parametrize("B,H,n", [(1, 40, 4096), (1, 33, 2100), (2, 36, 1100)])
def test_workgroups_walking_several_tiles(dev, B, H, n):
    """d = 128 bf16 without the mask and with more 256-row tiles than compute
    units: each workgroup walks tiles w, w + grid, ..., loading the next
    tile while it writes the current one, some workgroups one tile more
    than others (640, 297 and 360 tiles on 256 compute units; ragged row
    counts).  Every head is computed by some workgroup's first, second or
    third tile: the first, a middle and the last head against the oracle,
    and every head bitwise equal to calls on slices of heads small enough
    for one tile per workgroup on the same kernel (more than 128 and at most
    256 tiles)."""
    d = 128
    q, k, v = workloads.random_qkv(7300 + n + H, B, H, n, n, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.forward(qd, kd, vd, scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H // 2), (B - 1, H - 1)):
        ro, rl = oracle.attention_fwd(np64(q[b, h]), np64(k[b, h]), np64(v[b, h]), scale, False)
        assert_close(f"O B{B} H{H} n{n} ({b},{h})", o[b, h].cpu(), ro, tol_for(torch.bfloat16))
        assert_close(f"LSE B{B} H{H} n{n} ({b},{h})", lse[b, h].cpu(), rl, TOL_LSE)
    tiles = -(-n // 256)
    per = 256 // tiles  # heads per slice: 129..256 tiles
    assert 128 < per * tiles <= 256
    for b in range(B):
        for h0 in range(0, H, per):
            h1 = min(H, h0 + per)
            if (h1 - h0) * tiles <= 128:
                h0 = max(0, h1 - per)
            o1, l1 = fa.forward(qd[b:b + 1, h0:h1].contiguous(), kd[b:b + 1, h0:h1].contiguous(),
                                vd[b:b + 1, h0:h1].contiguous(), scale=scale)
            assert torch.equal(o1[0], o[b, h0:h1]) and torch.equal(l1[0], lse[b, h0:h1]), f"heads {b},{h0}:{h1}"


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(dev, shape, causal, dtype, d):
    B, H, n_q, n_k = shape
    q, k, v = workloads.random_qkv(1000 + n_q * 7 + n_k + d, B, H, n_q, n_k, d, dtype)
    check_full(dev, q, k, v, 1.0 / math.sqrt(d), causal, f"{shape} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_values_all_ones_gives_ones(dev, dtype):
    # The probabilities of each row sum to one, so V = 1 gives O = 1.
    q, k, _ = workloads.random_qkv(5, 1, 2, 300, 300, 64, dtype)
    v = torch.ones(1, 2, 300, 64, dtype=dtype)
    for causal in (False, True):
        o, _ = run_fwd(dev, q, k, v, 0.125, causal)
        assert_close("O (V=1)", o, np.ones(o.shape), 1e-6 if dtype == torch.float32 else 4e-3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_queries_give_prefix_means(dev, dtype):
    _, k, v = workloads.random_qkv(6, 1, 1, 200, 200, 32, dtype)
    q = torch.zeros(1, 1, 200, 32, dtype=dtype)
    vv = np64(v[0, 0])
    for causal in (False, True):
        o, lse = run_fwd(dev, q, k, v, 0.2, causal)
        cnt = np.arange(1, 201) if causal else np.full(200, 200)
        ref = np.cumsum(vv, axis=0) / cnt[:, None] if causal else np.broadcast_to(vv.mean(0), (200, 32))
        assert_close("O (Q=0)", o[0, 0], ref, tol_for(dtype))
        assert_close("LSE (Q=0)", lse[0, 0], np.log(cnt), TOL_LSE)


def test_scale_zero_is_uniform(dev):
    q, k, v = workloads.random_qkv(7, 1, 1, 130, 150, 64, torch.float32)
    for causal in (False, True):
        o, lse = run_fwd(dev, q, k, v, 0.0, causal)
        ro, rl = oracle.attention_fwd(np64(q), np64(k), np64(v), 0.0, causal)
        assert_close("O scale 0", o, ro, 1e-5)
        assert_close("LSE scale 0", lse, rl, TOL_LSE)


def test_causal_first_row_and_future_independence(dev):
    q, k, v = workloads.random_qkv(8, 1, 1, 256, 256, 128, torch.bfloat16)
    o, lse = run_fwd(dev, q, k, v, 1 / math.sqrt(128), True)
    assert torch.equal(o[0, 0, 0], v[0, 0, 0])
    ref0 = float((np64(q[0, 0, 0]) @ np64(k[0, 0, 0])) / math.sqrt(128))
    assert abs(float(lse[0, 0, 0]) - ref0) < TOL_LSE
    # Changing keys/values after row i leaves rows <= i bitwise unchanged.
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 130:] = 3.0
    v2[:, :, 130:] = -7.0
    o2, lse2 = run_fwd(dev, q, k2, v2, 1 / math.sqrt(128), True)
    assert torch.equal(o2[:, :, :130], o[:, :, :130])
    assert torch.equal(lse2[:, :, :130], lse[:, :, :130])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_online_softmax_stress(dev, dtype):
    n, d = 512, 64
    # Scores rising along the keys: the running max moves in every block.
    q = torch.ones(1, 1, n, d)
    k = (torch.arange(n, dtype=torch.float32) / 64.0)[:, None].expand(n, d).reshape(1, 1, n, d).contiguous()
    v = workloads.random_qkv(9, 1, 1, n, n, d, torch.float32)[2]
    # A planted late spike in another head, and very negative scores in a third.
    q2, k2, v2 = workloads.random_qkv(10, 1, 3, n, n, d, torch.float32)
    k2[0, 0] = k[0, 0]
    q2[0, 0] = q[0, 0]
    k2[0, 1, n - 3] = q2[0, 1].mean(0) * 40.0
    q2[0, 2] = -q2[0, 2].abs() * 3.0
    k2[0, 2] = k2[0, 2].abs() * 3.0
    v2[0, 0] = v[0, 0]
    q2, k2, v2 = (t.to(dtype) for t in (q2, k2, v2))
    # Scores here reach magnitudes near 50, far from N(0, 1): the fp32 bound
    # follows the rounding of those dot products.
    tol = fp32_score_tol(q2, k2, v2, 1 / math.sqrt(d)) if dtype == torch.float32 else None
    for causal in (False, True):
        check_full(dev, q2, k2, v2, 1 / math.sqrt(d), causal, f"stress causal={causal}", tol=tol)


def test_large_magnitude_inputs(dev):
    q, k, v = workloads.random_qkv(11, 1, 2, 300, 300, 128, torch.bfloat16, std=8.0)
    for causal in (False, True):
        check_full(dev, q, k, v, 1 / math.sqrt(128), causal, "std 8")


# bf16 on the d = 128 kernels; fp32 with few row blocks and 1500 keys on the
# eight-wave 16-row key-split kernel (its merge order is fixed)
@pytest.mark.parametrize("B,H,n,d,dtype", [(2, 4, 777, 128, torch.bfloat16), (1, 2, 1500, 64, torch.float32)],
                         ids=["bf16", "fp32_key_split"])
def test_repeatable_bitwise(dev, B, H, n, d, dtype):
    q, k, v = workloads.random_qkv(12, B, H, n, n, d, dtype)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for causal in (False, True):
        a = fa.forward(qd, kd, vd, causal=causal)
        b = fa.forward(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,H,n", [(torch.bfloat16, 3, 200), (torch.float32, 3, 200), (torch.float32, 2, 1500)],
                         ids=["bf16", "fp32", "fp32_eight_wave_key_split"])
def test_writes_stay_in_bounds(dev, dtype, H, n):
    # Outputs are views into larger buffers filled with a canary value.
    B, d = 1, 64
    q, k, v = (t.to(dev) for t in workloads.random_qkv(13, B, H, n, n, d, dtype))
    pad = 4096
    ob = torch.full((pad + B * H * n * d + pad,), 1234.0, dtype=dtype, device=dev)
    lb = torch.full((pad + B * H * n + pad,), 1234.0, dtype=torch.float32, device=dev)
    o = ob[pad:pad + B * H * n * d].view(B, H, n, d)
    lse = lb[pad:pad + B * H * n].view(B, H, n)
    fa.forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(ob[:pad] == 1234.0) and torch.all(ob[-pad:] == 1234.0)
    assert torch.all(lb[:pad] == 1234.0) and torch.all(lb[-pad:] == 1234.0)
    assert torch.all(torch.isfinite(o))


def test_no_score_matrix_allocation(dev):
    # The library allocates nothing: device memory in use does not grow
    # during a call at a size whose score matrix would be 1 GiB in bf16.
    w = workloads.c3(False)
    q, k, v = w.q[:, :16].contiguous().to(dev), w.k[:, :16].contiguous().to(dev), w.v[:, :16].contiguous().to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    fa.forward(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 < 64 * 1024 * 1024
