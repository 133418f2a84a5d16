"""Throughput of one exact-attention training step on one MI355X.

A step is the whole path once: the forward pass (O and LSE) and the
recomputation backward pass (delta = rowsum(dO o O), then dK/dV, then dQ) on
B=1, H=32, n=4096, d=128 bf16 inputs already resident in device memory, each
stage called through the C ABI on the current stream.

value      = algorithmic FLOP of the step / step time, in TFLOP/s:
             forward 4*B*H*n^2*d, backward 10*B*H*n^2*d (five products per
             visible query-key pair); the causal variant counts only visible
             pairs.
roofline   = the kernel taking the largest share of the step, its algorithmic
             FLOP per launch over its mean launch time from HIP events recorded
             around it inside the timed loop, against the bf16 dense
             matrix-core peak.
cpu_baseline = the fp64 oracle timed on a bounded sample of the same workload,
             with the CPU model and the BLAS library (vendor, threads).
flops      = each pass counted two ways: literal 4*B*H*n^2*d and algorithmic
             (visible pairs, 2 products forward, 5 backward).

--workload configs times each workload's hot call, one ring-attention step
(fa_forward_merge against fa_forward + fa_lse_merge) and, unless
--no-cpu-baseline, the fp64 oracle on every workload.

With --workload decode the step is instead one split-KV decoding call
(fa_decode: 4 sequences x 64 query heads over 8 K/V heads, one new query row
each, 32768 cached keys, d=128, bf16), an HBM-bound pass: value is the
algorithmic bytes (K and V read once, q read, o and lse written) over the
call time in GB/s, and the roofline is against HBM bandwidth.

One JSON line is printed.  Only one GPU is supported: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix cores
PEAK_HBM_GBS = 8000.0
PEAK_SCLK_MHZ = 2400.0      # shader clock the peak figures assume
METRIC = "attention fwd/bwd TFLOP/s (4·B·H·n²·d/t) and % bf16 MFMA peak at n=4096,d=128"

KERNEL_SOURCES = {
    "decode": "exact_attention_05_amd/csrc/fa_decode.hip",
    "fwd": "exact_attention_05_amd/csrc/fa_fwd.hip",
    "bwd_preprocess": "exact_attention_05_amd/csrc/fa_bwd.hip",
    "bwd_dkdv": "exact_attention_05_amd/csrc/fa_bwd.hip",
    "bwd_dq": "exact_attention_05_amd/csrc/fa_bwd.hip",
}


def visible_pairs(n_q: int, n_k: int, causal: bool) -> int:
    if not causal:
        return n_q * n_k
    m = min(n_q, n_k)
    # rows 0..m-1 see i+1 keys; rows m..n_q-1 see all n_k keys
    return m * (m + 1) // 2 + (n_q - m) * n_k


def kernel_flops(B, H, n, d, causal):
    """Algorithmic FLOP per launch of each stage (what the method must do)."""
    pairs = B * H * visible_pairs(n, n, causal)
    return {
        "fwd": 4 * d * pairs,             # S = QK^T and P V
        "bwd_preprocess": 2 * B * H * n * d,
        "bwd_dkdv": 8 * d * pairs,        # S recomputed, dP, dV, dK
        "bwd_dq": 2 * d * pairs,          # dQ (its S, dP recompute is overhead)
    }


def kernel_bytes(B, H, n, d, e=2):
    """Algorithmic HBM bytes per launch (each operand read once, results written once)."""
    t = B * H * n * d * e
    r = B * H * n * 4
    return {
        "fwd": 3 * t + t + r,                     # read q k v, write o lse
        "bwd_preprocess": 2 * t + 3 * r,          # read o dO lse, write delta and lse*log2(e)
        "bwd_dkdv": 4 * t + 2 * r + 2 * t,        # read q k v dO lse delta, write dk dv
        "bwd_dq": 4 * t + 2 * r + t,              # read q k v dO lse delta, write dq
    }


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE,
    if recorded for the current source of that kernel on this workload (the
    tag of the profile summary); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def kernel_source_digest(kernel: str) -> str:
    """sha256 over the kernel's .hip file and every header it can include."""
    csrc = os.path.join(ROOT, "exact_attention_05_amd", "csrc")
    h = hashlib.sha256()
    files = [os.path.join(ROOT, KERNEL_SOURCES[kernel])]
    files += sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hpp"))
    files.append(os.path.join(ROOT, "include", "fa.h"))
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def host_info():
    """What the CPU figures ran on: the CPU model (/proc/cpuinfo), the cores
    this process may use, and the BLAS library numpy calls (vendor, version,
    threads)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl

        for i in threadpoolctl.threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "library": os.path.basename(i.get("filepath") or "")}
                break
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)), "blas": blas}


def _f64(torch_tensor):
    import numpy as np

    return torch_tensor.float().numpy().astype(np.float64)


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle (forward + explicit backward) on whole (b, h) units of
    the same workload, repeated until about ``budget_s`` seconds of CPU work."""
    import oracle

    host = host_info()
    B, H, n, d = w.q.shape
    units = [(0, h) for h in range(H)]
    t0 = time.perf_counter()
    done = 0
    while done < len(units):
        b, h = units[done]
        q, k, v, do = (_f64(x[b, h]) for x in (w.q, w.k, w.v, w.do))
        oracle.attention_fwd(q, k, v, w.scale, w.causal)
        oracle.attention_bwd(q, k, v, do, w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = done * 14 * d * visible_pairs(n, n, w.causal)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": (host["blas"] or {}).get("threads"),
        "kind": "oracle",
        "sample": f"{done} of {B * H} (b,h) units, fp64 numpy forward + explicit backward, {dt:.1f} s",
        "cpu_model": host["cpu_model"],
        "cores_available": host["cores_available"],
        "blas": host["blas"],
    }


def cpu_oracle_configs(workloads, log):
    """The fp64 oracle timed on every workload (baseline only, never a
    target): c1-c3 the full forward, c4 the 256 checked rows plus one full
    head (x32, an extrapolation), c5 the full forward + explicit backward.
    TFLOP/s use the GPU's algorithmic counts."""
    import oracle

    res = {"host": host_info()}

    def fwd_full(name, w):
        B, H, n, d = w.q.shape
        t0 = time.perf_counter()
        for b in range(B):
            for h in range(H):
                oracle.attention_fwd(_f64(w.q[b, h]), _f64(w.k[b, h]), _f64(w.v[b, h]), w.scale, w.causal)
        dt = time.perf_counter() - t0
        fl = 4 * d * B * H * visible_pairs(n, n, w.causal)
        res[name] = {"s": round(dt, 3), "tflops": round(fl / dt / 1e12, 6), "scope": "full forward"}
        log(f"cpu oracle {name}: {dt:.1f} s")

    fwd_full("c1", workloads.c1())
    fwd_full("c2", workloads.c2())
    fwd_full("c3_noncausal", workloads.c3(False))
    fwd_full("c3_causal", workloads.c3(True))

    w = workloads.c4()
    B, H, n, d = w.q.shape
    qf, kf, vf = (_f64(x) for x in (w.q, w.k, w.v))
    t0 = time.perf_counter()
    oracle.attention_rows(qf, kf, vf, workloads.c4_rows(), w.scale, True)
    t_rows = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attention_fwd(qf[0, 0], kf[0, 0], vf[0, 0], w.scale, True)
    t_head = time.perf_counter() - t0
    del qf, kf, vf
    fl = 4 * d * B * H * visible_pairs(n, n, True)
    res["c4_causal"] = {"s_256_rows": round(t_rows, 3), "s_one_head": round(t_head, 3),
                        "s_full_extrapolated": round(32 * t_head, 2),
                        "tflops": round(fl / (32 * t_head) / 1e12, 6),
                        "scope": "256 checked rows timed; one full head timed, x32 extrapolation"}
    log(f"cpu oracle c4: rows {t_rows:.1f} s, one head {t_head:.1f} s")
    del w

    w = workloads.c5()
    B, H, n, d = w.q.shape
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            q, k, v, do = (_f64(x[b, h]) for x in (w.q, w.k, w.v, w.do))
            oracle.attention_fwd(q, k, v, w.scale, True)
            oracle.attention_bwd(q, k, v, do, w.scale, True)
    dt = time.perf_counter() - t0
    pairs = B * H * visible_pairs(n, n, True)
    res["c5_fwd_bwd_causal"] = {"s": round(dt, 3), "tflops": round(14 * d * pairs / dt / 1e12, 6),
                                "scope": "full forward + explicit backward"}
    log(f"cpu oracle c5: {dt:.1f} s")
    return res


def calibration_copy(torch, dev):
    """One elementwise copy of 512 MiB (fp32 x*1 into a second buffer): a
    kernel of known traffic for scaling the memory counters."""
    src = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def decode_bytes(B, H, H_kv, n_q, n_k, d, e=2):
    """Algorithmic HBM bytes of one decoding call: K and V read once, q read,
    o and lse written (the chunk partials are overhead)."""
    return 2 * B * H_kv * n_k * d * e + 2 * B * H * n_q * d * e + B * H * n_q * 4


def cpu_baseline_decode(w, budget_s: float):
    """The fp64 oracle (banded forward) on whole (b, h) units of the decoding
    workload until about ``budget_s`` seconds of CPU work; reported as K/V
    bytes processed per second, like the GPU value."""
    import numpy as np

    import oracle

    B, H, n_q, d = w.q.shape
    h_kv, n_k = w.k.shape[1], w.k.shape[2]
    group = H // h_kv
    t0 = time.perf_counter()
    done = 0
    for b in range(B):
        for j in range(h_kv):
            k = w.k[b, j].float().numpy().astype(np.float64)
            v = w.v[b, j].float().numpy().astype(np.float64)
            for h in range(j * group, (j + 1) * group):
                q = w.q[b, h].float().numpy().astype(np.float64)
                oracle.attention_fwd_band(q, k, v, w.scale, True, n_k - n_q)
                done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_unit = decode_bytes(B, H, h_kv, n_q, n_k, d) / (B * H)
    return {
        "value": done * per_unit / dt / 1e9,
        "unit": "GB/s",
        "cores": None,
        "kind": "oracle",
        "sample": f"{done} of {B * H} (b,h) query heads, fp64 numpy banded forward over {n_k} keys, {dt:.1f} s",
    }


def run_decode(args, torch, fa, workloads, dev):
    w = workloads.decode_gqa()
    B, H, n_q, d = w.q.shape
    h_kv, n_k = w.k.shape[1], w.k.shape[2]
    q, k, v = (t.to(dev).contiguous() for t in (w.q, w.k, w.v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    splits = fa.decode_splits(B, H, h_kv, n_q, n_k)
    ws = torch.empty(max(1, fa.decode_workspace_size(B, H, n_q, d, splits)), dtype=torch.uint8, device=dev)
    steps = args.steps if args.steps is not None else 200   # a call is ~0.1 ms: time more of them
    warmup = args.warmup if args.warmup is not None else 1000  # ~0.1 s: let the clock settle

    def step():
        fa.decode(q, k, v, causal=True, scale=w.scale, n_splits=splits, out=o, lse=lse, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in events:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.calibration_copy:
        calibration_copy(torch, dev)
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in events) / steps
    ms_per_step = wall * 1e3 / steps
    nbytes = decode_bytes(B, H, h_kv, n_q, n_k, d)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    out = {
        "metric": "split-KV decoding: algorithmic HBM GB/s (K, V read once) at 32K context",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v; no dataset)",
        "config": {"workload": w.name, "B": B, "H": H, "H_kv": h_kv, "n_q": n_q, "n_k": n_k, "d": d,
                   "causal": True, "q_offset": n_k - n_q, "n_splits": splits,
                   "step": "fa_decode (decode kernel + chunk merge)"},
        "kernels": {"decode": {"ms": round(call_ms, 4), "gbs": round(achieved, 1)}},
        "roofline": {
            "kernel": "decode",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("decode", f"decode_b{B}h{H}hkv{h_kv}_nk{n_k}_d{d}"),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_budget)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 3)
        try:
            import threadpoolctl

            info = threadpoolctl.threadpool_info()
            out["cpu_baseline"]["cores"] = max([i.get("num_threads", 1) for i in info
                                                if i.get("user_api") == "blas"] or [1])
        except Exception:  # noqa: BLE001
            pass
    print(json.dumps(out), flush=True)
    return 0


PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 matrix / vector peak


def _median_us(torch, fn, reps: int, warmup: int = 3, batch: int = 10, settle_s: float = 0.3):
    """Per-call time of fn() in microseconds: the median over ``reps`` HIP-event
    measurements of ``batch`` back-to-back calls each (calls issued one at a
    time with an idle GPU in between run at a lower clock), after at least
    ``warmup`` calls and ``settle_s`` seconds of back-to-back calls, so that
    the shader clock has settled under the load."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(batch):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / batch)
    ts.sort()
    return ts[len(ts) // 2]


def _sclk_sampler():
    """Best-effort sampling of the GPU's shader clock (amd-smi) in a thread;
    returns (start, stop, count) where stop(t0, t1) gives the mean MHz of the
    samples taken entirely inside [t0, t1] (perf_counter times) or None, and
    count(t0) the number of samples completed that began at or after t0 (-1
    when amd-smi is missing or failed)."""
    import subprocess
    import threading

    samples, done = [], threading.Event()

    def run():
        while not done.is_set():
            try:
                t_a = time.perf_counter()
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                                   capture_output=True, text=True, timeout=5)
                t_b = time.perf_counter()
                data = json.loads(r.stdout)
                node = data["gpu_data"][0] if isinstance(data, dict) and "gpu_data" in data else (
                    data[0] if isinstance(data, list) else data)
                clk = node.get("clock", {})
                vals = [float(v["clk"]["value"]) for k, v in clk.items()
                        if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                        and v["clk"].get("value") not in (None, "N/A")]
                if vals:
                    samples.append((t_a, t_b, sum(vals) / len(vals)))  # mean over the XCDs
            except Exception:  # noqa: BLE001
                return
            done.wait(0.05)

    t = threading.Thread(target=run, daemon=True)

    def stop(t0=float("-inf"), t1=float("inf")):
        done.set()
        t.join(timeout=10)
        inside = [v for a, b, v in samples if a >= t0 and b <= t1]
        return round(sum(inside) / len(inside), 1) if inside else None

    def count(t0):
        """Samples begun at or after t0; -1 once the sampler has given up."""
        if not t.is_alive():
            return -1
        return sum(1 for a, _, _ in list(samples) if a >= t0)

    return t.start, stop, count


def _sclk_under_load(launch, torch, settle_s=1.5, min_s=1.0, max_s=8.0, want=3):
    """Mean shader clock (MHz) over amd-smi samples taken while `launch()`
    (a batch of GPU work) runs back to back.  The amdgpu kernel module refreshes the value
    about once a second, so samples are only counted after settle_s seconds
    of load, for at least min_s more seconds and until `want` of them are
    in, or max_s seconds of load in all."""
    start, stop, count = _sclk_sampler()
    start()
    launch()
    torch.cuda.synchronize()  # the GPU is busy from here on
    t_busy = time.perf_counter()
    t0 = t_busy + settle_s
    while True:
        launch()
        torch.cuda.synchronize()
        now = time.perf_counter()
        c = count(t0)
        if c < 0 or now - t_busy >= max_s or (now >= t0 + min_s and c >= want):
            break
    return stop(t0, time.perf_counter())


def run_configs(args, torch, fa, workloads, dev):
    """Each workload's hot call timed on its own (median of HIP-event times),
    plus the short-sequence HBM sweep of the forward pass."""
    res = {}

    def fwd_entry(w, reps=10):
        q, k, v = (t.to(dev).contiguous() for t in (w.q, w.k, w.v))
        o = torch.empty_like(q)
        B, H, n, d = q.shape
        lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        us = _median_us(torch, lambda: fa.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse), reps)
        flops = 4 * d * B * H * visible_pairs(n, n, w.causal)
        peak = PEAK_BF16_TFLOPS if q.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
        tf = flops / (us * 1e-6) / 1e12
        entry = {"us": round(us, 1), "tflops": round(tf, 2), "pct_peak": round(100 * tf / peak, 2),
                 "peak": peak}
        if w.causal:
            entry["tflops_literal"] = round(4 * d * B * H * n * n / (us * 1e-6) / 1e12, 2)
        return entry

    res["c1"] = fwd_entry(workloads.c1())
    res["c2_fp32"] = fwd_entry(workloads.c2(torch.float32))
    res["c2_bf16"] = fwd_entry(workloads.c2(torch.bfloat16))
    # c2 has one head: 16 query tiles for 256 compute units.  The split-KV
    # entry point (fa_decode) spreads the keys over more workgroups.
    w2 = workloads.c2(torch.bfloat16)
    q2, k2, v2 = (t.to(dev) for t in (w2.q, w2.k, w2.v))
    o2 = torch.empty_like(q2)
    l2 = torch.empty(q2.shape[:3], dtype=torch.float32, device=dev)
    sp = fa.decode_splits(1, 1, 1, q2.shape[2], k2.shape[2])
    ws2 = torch.empty(max(1, fa.decode_workspace_size(1, 1, q2.shape[2], q2.shape[3], sp)),
                      dtype=torch.uint8, device=dev)
    us = _median_us(torch, lambda: fa.decode(q2, k2, v2, causal=False, q_offset=0, scale=w2.scale,
                                              n_splits=sp, out=o2, lse=l2, workspace=ws2), 10)
    tf = 4 * 64 * 4096 * 4096 / (us * 1e-6) / 1e12
    res["c2_bf16_split_kv"] = {"us": round(us, 1), "tflops": round(tf, 2),
                               "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "n_splits": sp}
    del q2, k2, v2, o2, l2, ws2
    res["c3_noncausal"] = fwd_entry(workloads.c3(False))
    # the shader clock while the c3 forward runs back to back
    w3 = workloads.c3(False)
    q3, k3, v3 = (t.to(dev) for t in (w3.q, w3.k, w3.v))

    def c3_batch():
        for _ in range(40):
            fa.forward(q3, k3, v3, scale=w3.scale)

    sclk = _sclk_under_load(c3_batch, torch)
    del q3, k3, v3
    res["c3_causal"] = fwd_entry(workloads.c3(True))
    res["c4_causal"] = fwd_entry(workloads.c4(), reps=5)
    torch.cuda.empty_cache()
    # c5: the backward pass (three stages) after one forward.
    w = workloads.c5()
    q, k, v, do = (t.to(dev).contiguous() for t in (w.q, w.k, w.v, w.do))
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    ws = fa.backward_workspace(*q.shape[:3], k.shape[2], q.shape[3], q.dtype, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    us = _median_us(torch, lambda: fa.backward(q, k, v, o, do, lse, causal=True, scale=w.scale,
                                                dq=dq, dk=dk, dv=dv, workspace=ws), 10)
    B, H, n, d = q.shape
    pairs = B * H * visible_pairs(n, n, True)
    tf = 10 * d * pairs / (us * 1e-6) / 1e12
    res["c5_backward_causal"] = {"us": round(us, 1), "tflops": round(tf, 2),
                                 "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                                 "tflops_literal": round(4 * B * H * n * n * d / (us * 1e-6) / 1e12, 2)}
    del q, k, v, do, o, lse, ws, dq, dk, dv
    torch.cuda.empty_cache()

    # Per visible pair, how masked passes compare with full attention (B=1,
    # H=32, n=4096, d=128 bf16): forward and whole backward under no mask,
    # the causal mask, a +-256 window and a causal 512 window.
    def band_pairs(n, causal, window):
        tot = 0
        for i in range(n):
            lo, hi = 0, n - 1
            if causal:
                hi = min(hi, i)
            if window is not None:
                lo, hi = max(lo, i - window), min(hi, i + window)
            tot += max(0, hi - lo + 1)
        return tot

    wq = workloads.c3(False)
    q, k, v = (t.to(dev) for t in (wq.q, wq.k, wq.v))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(dev)
    B, H, n, d = q.shape
    ws = fa.backward_workspace(B, H, n, n, d, q.dtype, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    masks = {}
    for name, causal, window in (("full", False, None), ("causal", True, None), ("window256", False, 256),
                                 ("causal_window512", True, 512)):
        o, lse = fa.forward(q, k, v, causal=causal, window=window)
        uf = _median_us(torch, lambda: fa.forward(q, k, v, causal=causal, window=window, out=o, lse=lse), 10)
        ub = _median_us(torch, lambda: fa.backward(q, k, v, o, do, lse, causal=causal, window=window, dq=dq,
                                                    dk=dk, dv=dv, workspace=ws), 10)
        pairs = B * H * band_pairs(n, causal, window)
        masks[name] = {"fwd_us": round(uf, 1), "bwd_us": round(ub, 1), "pairs": pairs,
                       "fwd_tflops": round(4 * d * pairs / (uf * 1e-6) / 1e12, 1),
                       "bwd_tflops": round(10 * d * pairs / (ub * 1e-6) / 1e12, 1)}
    for name in masks:
        masks[name]["fwd_rate_vs_full"] = round(masks[name]["fwd_tflops"] / masks["full"]["fwd_tflops"], 3)
        masks[name]["bwd_rate_vs_full"] = round(masks[name]["bwd_tflops"] / masks["full"]["bwd_tflops"], 3)
    res["masks_b1h32n4096d128"] = masks
    del q, k, v, do, ws, dq, dk, dv, o, lse
    torch.cuda.empty_cache()

    # LSE merge of 8 bf16 parts of the c3 shape (the results of 8 key chunks,
    # as a sequence-sharded step combines them): HBM-bound, algorithmic bytes
    # = the parts (o and lse) read once and the result written once; 302 MB
    # per call, more than the 256 MB last-level cache.
    P, B, H, n, d = 8, 1, 32, 4096, 128
    g = torch.Generator(device="cpu").manual_seed(8)
    o_parts = torch.randn(P, B, H, n, d, generator=g).to(torch.bfloat16).to(dev)
    lse_parts = (torch.randn(P, B, H, n, generator=g) * 2.0).to(dev)
    mo = torch.empty((B, H, n, d), dtype=torch.bfloat16, device=dev)
    ml = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    us = _median_us(torch, lambda: fa.lse_merge(o_parts, lse_parts, out=mo, lse=ml), 20)
    nbytes = P * B * H * n * (d * 2 + 4) + B * H * n * (d * 2 + 4)
    res["merge8_c3_bf16"] = {"us": round(us, 1), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "pct_hbm": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)}
    del o_parts, lse_parts, mo, ml
    torch.cuda.empty_cache()

    # One ring-attention step at the c3 shape: 4096 local query rows of 32
    # heads take a 4096-key chunk and fold it into the running (O, LSE).
    # Fused: fa_forward_merge, one launch.  Separate: fa_forward into a part,
    # then fa_lse_merge of (running, part), whose O makes a round trip
    # through HBM.  Out of place (the running result is double-buffered).
    w3 = workloads.c3(False)
    q3, k3, v3 = (t.to(dev) for t in (w3.q, w3.k, w3.v))
    B, H, n, d = q3.shape
    g = torch.Generator(device="cpu").manual_seed(16)
    ring = {}
    for acc in (torch.bfloat16, torch.float32):
        o_run = torch.randn(B, H, n, d, generator=g).to(acc).to(dev)
        l_run = (torch.randn(B, H, n, generator=g) * 2.0 + 8.0).to(dev)
        o_new, l_new = torch.empty_like(o_run), torch.empty_like(l_run)
        us = _median_us(torch, lambda: fa.forward_merge(q3, k3, v3, o_run, l_run, scale=w3.scale,
                                                          out=o_new, lse=l_new), 10)
        ring[f"fused_{str(acc).split('.')[-1]}_running_o_us"] = round(us, 1)
    parts = torch.empty((2, B, H, n, d), dtype=torch.bfloat16, device=dev)
    lparts = torch.empty((2, B, H, n), dtype=torch.float32, device=dev)
    parts[0] = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16).to(dev)
    lparts[0] = (torch.randn(B, H, n, generator=g) * 2.0 + 8.0).to(dev)
    mo = torch.empty((B, H, n, d), dtype=torch.bfloat16, device=dev)
    ml = torch.empty((B, H, n), dtype=torch.float32, device=dev)

    def separate():
        fa.forward(q3, k3, v3, scale=w3.scale, out=parts[1], lse=lparts[1])
        fa.lse_merge(parts, lparts, out=mo, lse=ml)

    ring["separate_bf16_running_o_us"] = round(_median_us(torch, separate, 10), 1)
    ring["saved_pct_bf16"] = round(100 * (1 - ring["fused_bfloat16_running_o_us"]
                                          / ring["separate_bf16_running_o_us"]), 1)
    res["ring_step_c3_chunk4096"] = ring
    del q3, k3, v3, o_run, l_run, o_new, l_new, parts, lparts, mo, ml
    torch.cuda.empty_cache()

    # Short-sequence sweep: B=16, H=32, d=128 bf16 non-causal forward, input
    # sets rotated so that the bytes touched between two calls of the same
    # set exceed the 256 MB last-level cache.
    sweep = {}
    for n in (128, 256, 512, 1024):
        B, H, d = 16, 32, 128
        per_set = 4 * B * H * n * d * 2
        sets = max(3, -(-768 * 2**20 // per_set))
        bufs = []
        g = torch.Generator(device="cpu").manual_seed(n)
        for _ in range(sets):
            t = torch.randn(3, B, H, n, d, generator=g).to(torch.bfloat16).to(dev)
            bufs.append((t[0], t[1], t[2], torch.empty((B, H, n, d), dtype=torch.bfloat16, device=dev),
                         torch.empty((B, H, n), dtype=torch.float32, device=dev)))
        it = [0]

        def call():
            qq, kk, vv, oo, ll = bufs[it[0] % sets]
            it[0] += 1
            fa.forward(qq, kk, vv, out=oo, lse=ll)

        us = _median_us(torch, call, 20, warmup=sets)
        nbytes = 4 * B * H * n * d * 2 + 4 * B * H * n
        sweep[f"n{n}"] = {"us": round(us, 1), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "pct_hbm": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
                          "tflops": round(4 * d * B * H * n * n / (us * 1e-6) / 1e12, 2)}
        del bufs
        torch.cuda.empty_cache()

    out = {
        "metric": "per-workload hot-call throughput (TFLOP/s algorithmic, % of the dtype's peak)",
        "value": res["c3_noncausal"]["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 3,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1); no dataset)",
        "config": {"workload": "c1..c5 hot calls + short-sequence HBM sweep (B16 H32 d128)"},
        "configs": res,
        "hbm_sweep": sweep,
        "sclk_mhz_mean_c3_forward": sclk,
    }
    if not args.no_cpu_baseline:
        out["cpu_oracle"] = cpu_oracle_configs(workloads, lambda m: print(m, file=sys.stderr, flush=True))
    print(json.dumps(out), flush=True)
    return 0


# ------------------------------------------------ profiler summaries
# rocprofv3 writes CSV files (kernel trace, kernel stats, counter
# collection); these turn them into the short summaries kept under profiles/
# and the per-kernel traffic records load_traffic() reads.

STAGE_PATTERNS = [("bwd_preprocess", "bwd_preprocess"), ("bwd_dkdv", "bwd_dkdv"), ("bwd_dq", "bwd_dq"),
                  ("bwd_reduce", "bwd_reduce_slices"), ("decode", "decode_bf16"), ("lse_merge", "lse_merge"),
                  ("fwd", "fwd_")]
COPY_KIB = 512 * 1024  # the calibration copy reads and writes 512 MiB


def stage_of(kernel_name: str):
    """The library stage a profiled kernel belongs to, from its (demangled or
    mangled) name; None for kernels outside the library, such as torch's."""
    for stage, pat in STAGE_PATTERNS:
        if pat in kernel_name:
            return stage
    return None


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counter_per_dispatch(directory: str, counter: str):
    """{kernel name: [value per dispatch, in dispatch order]} for one counter."""
    per = {}
    rows = [r for r in _csv_rows(directory, "counter_collection.csv") if r.get("Counter_Name") == counter]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def _copy_kernel(fetch: dict):
    """The calibration copy: the non-library kernel that read the most (the
    fill that creates its source writes as much but reads nothing)."""
    cands = {k: max(v) for k, v in fetch.items() if stage_of(k) is None}
    return max(cands, key=cands.get)


def record_traffic(fetch_dir: str, write_dir: str, tag: str, commands: list[str]) -> str:
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    copy_f = _copy_kernel(fetch)
    copy_w = copy_f
    ff = COPY_KIB / max(fetch[copy_f])
    wf = COPY_KIB / max(write[copy_w])
    lines = [f"# HBM traffic counters: {tag}", "",
             "Commands (from the repository root, on one MI355X; two separate counter runs, then this summary):",
             "", "```", "export TMPDIR=/tmp", *commands, "```", "",
             "Calibration: the elementwise copy run by --calibration-copy reads and writes exactly 512 MiB "
             f"({COPY_KIB} KiB).",
             f"Its FETCH_SIZE reads {max(fetch[copy_f]):.0f} KiB and WRITE_SIZE {max(write[copy_w]):.0f} KiB, "
             f"so the scale factors are fetch x{ff:.3f}, write x{wf:.3f}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | scaled HBM bytes/launch |",
             "|---|---|---|---|---|"]
    for name in sorted(fetch, key=lambda k: (stage_of(k) is None, str(stage_of(k)), k)):
        stage = stage_of(name)
        if stage is None or name not in write:
            continue
        # the last dispatches are the timed ones; the first may run on cold caches
        fk = fetch[name][-1]
        wk = write[name][-1]
        nbytes = int(round((fk * ff + wk * wf) * 1024))
        lines.append(f"| {stage}: `{name[:90]}` | {len(fetch[name])} | {fk:.0f} | {wk:.0f} | {nbytes} |")
        src = KERNEL_SOURCES.get(stage)
        if src:
            rec = {"kernel": stage, "kernel_name": name, "workload": tag, "source": src,
                   "source_sha256": kernel_source_digest(stage), "fetch_kib": fk, "write_kib": wk,
                   "fetch_factor": ff, "write_factor": wf, "bytes_per_launch": nbytes,
                   "summary": f"profiles/traffic_{tag}.md"}
            with open(os.path.join(ROOT, "profiles", f"traffic_{stage}.json"), "w") as f:
                json.dump(rec, f, indent=1)
    lines.append(f"| copy 512 MiB: `{copy_w[:90]}` | 1 | {max(fetch[copy_f]):.0f} | {max(write[copy_w]):.0f} | "
                 f"{2 * COPY_KIB * 1024} |")
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def summarize_trace(trace_dir: str, tag: str, commands: list[str], timed: int, note: str) -> str:
    """Per-kernel calls, mean/min/max and share from the kernel stats, plus
    the mean of the last ``timed`` dispatches of each kernel from the trace."""
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    durs = {}
    for r in sorted(trace, key=lambda r: int(r.get("Start_Timestamp") or 0)):
        durs.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# Kernel trace: {tag}", "", "Command (from the repository root, on one MI355X), then this summary:",
             "", "```", "export TMPDIR=/tmp", *commands, "```", "", note, "",
             "| kernel | calls | mean us | min us | max us | share | mean us of the timed calls |",
             "|---|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        d = durs.get(name, [])
        last = d[-timed:] if timed else d
        tail = f"{sum(last) / len(last):.1f} (last {len(last)})" if last else "-"
        lines.append(f"| `{name[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% | {tail} |")
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def summarize_counters(dirs: list[str], tag: str, commands: list[str]) -> str:
    """SQ/GRBM counter passes (one directory each) -> per-kernel means and the
    derived figures: MFMA utilisation at the running clock, vector and LDS
    instructions per product, co-issue and LDS-wait cycles per SIMD."""
    simds, xcds = 1024, 8
    per = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            stage = stage_of(r["Kernel_Name"])
            if stage is None:
                continue
            per.setdefault(stage, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    lines = [f"# Counters: {tag}", "", "Commands (from the repository root, on one MI355X; one counter pass per run), "
             "then this summary:", "", "```", "export TMPDIR=/tmp", *commands, "```", "",
             f"Mean per launch.  SQ counters are summed over the {simds} SIMDs, GRBM_GUI_ACTIVE over the {xcds} XCDs.  "
             "Each 32x32x16 bf16 product adds 32 to SQ_VALU_MFMA_BUSY_CYCLES, so MFMA utilisation at the running "
             "clock = (MFMA_BUSY / 1024) / (GRBM_GUI_ACTIVE / 8).  SQ_ACTIVE_INST_VALU and SQ_WAIT_INST_LDS count "
             "quad-cycles (x4 / 1024 per SIMD); co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / 1024.", "",
             "| kernel | MFMA instr | MFMA busy cyc/SIMD | GPU active cyc/XCD | MFMA util (running clock) | "
             "VALU instr / MFMA | VALU active cyc/SIMD | MFMA+VALU co-issue cyc/SIMD | LDS instr / MFMA | "
             "LDS bank conflicts | LDS-wait cyc/SIMD |", "|---|---|---|---|---|---|---|---|---|---|---|"]

    def g(m, c):
        return m.get(c, float("nan"))

    for k in sorted(mean):
        m = mean[k]
        mf = g(m, "SQ_INSTS_MFMA")
        busy = g(m, "SQ_VALU_MFMA_BUSY_CYCLES") / simds
        act = g(m, "GRBM_GUI_ACTIVE") / xcds
        ratio = (lambda a: a / mf if mf else float("nan"))
        lines.append(f"| {k} | {mf:.0f} | {busy:.0f} | {act:.0f} | {100 * busy / act:.1f} % | "
                     f"{ratio(g(m, 'SQ_INSTS_VALU')):.2f} | {4 * g(m, 'SQ_ACTIVE_INST_VALU') / simds:.0f} | "
                     f"{g(m, 'SQ_VALU_MFMA_COEXEC_CYCLES') / simds:.0f} | {ratio(g(m, 'SQ_INSTS_LDS')):.2f} | "
                     f"{g(m, 'SQ_LDS_BANK_CONFLICT'):.0f} | {4 * g(m, 'SQ_WAIT_INST_LDS') / simds:.0f} |")
    lines += ["", "Raw means:", "", "| kernel | counter | value |", "|---|---|---|"]
    for k in sorted(mean):
        for c in sorted(mean[k]):
            lines.append(f"| {k} | {c} | {mean[k][c]:.0f} |")
    path = os.path.join(ROOT, "profiles", f"counters_{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def profile_main(argv):
    """python bench.py summarize-trace DIR TAG TIMED NOTE CMD...
       python bench.py record-traffic FETCH_DIR WRITE_DIR TAG CMD...
       python bench.py summarize-counters DIR[,DIR...] TAG CMD..."""
    if argv[0] == "summarize-counters":
        print(summarize_counters(argv[1].split(","), argv[2], argv[3:]))
    elif argv[0] == "summarize-trace":
        print(summarize_trace(argv[1], argv[2], argv[5:], int(argv[3]), argv[4]))
    elif argv[0] == "record-traffic":
        print(record_traffic(argv[1], argv[2], argv[3], argv[4:]))
    else:
        raise SystemExit(profile_main.__doc__)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50 training steps, 200 decoding calls)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 100 training steps, 1000 decoding calls, "
                         "about 0.1 s, so that the timed steps run at the settled shader clock)")
    ap.add_argument("--workload", choices=["train", "decode", "configs"], default="train",
                    help="train: forward + backward at n=4096 (default); decode: split-KV decoding; "
                         "configs: every workload's hot call plus the short-sequence HBM sweep")
    ap.add_argument("--causal", action="store_true", help="causal mask (default: non-causal)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock (amd-smi) while the forward runs back to "
                         "back after the timed steps (about 3 s)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed steps, run one elementwise copy of 512 MiB (fp32 x*1 into "
                         "a second buffer) so that a counter run sees a kernel of known traffic")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange)", file=sys.stderr)
        return 2

    import torch

    import exact_attention_05_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.workload == "decode":
        return run_decode(args, torch, fa, workloads, dev)
    if args.steps is None:
        args.steps = 50
    if args.warmup is None:
        args.warmup = 100
    if args.workload == "configs":
        return run_configs(args, torch, fa, workloads, dev)
    w = workloads.c3_train(args.causal)
    B, H, n, d = w.q.shape
    q, k, v, do = (t.to(dev).contiguous() for t in (w.q, w.k, w.v, w.do))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    ws = fa.backward_workspace(B, H, n, n, d, q.dtype, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    causal = args.causal

    stages = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.backward_preprocess(o, do, lse, ws)
        if ev is not None:
            ev[2].record()
        fa.backward_dkdv(q, k, v, do, ws, causal=causal, scale=w.scale, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record()
        fa.backward_dq(q, k, v, do, ws, causal=causal, scale=w.scale, dq=dq)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    sclk = None
    if not args.no_clock:
        # Outside the timed region: the mean shader clock while the forward
        # runs back to back, to state the peak fraction at the running clock.
        def fwd_batch():
            for _ in range(40):
                fa.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)

        sclk = _sclk_under_load(fwd_batch, torch)

    if args.calibration_copy:
        calibration_copy(torch, dev)

    per_stage = {s: 0.0 for s in stages}
    step_ms = []
    for ev in events:
        for j, s in enumerate(stages):
            per_stage[s] += ev[j].elapsed_time(ev[j + 1])
        step_ms.append(ev[0].elapsed_time(ev[4]))
    per_stage = {s: t / args.steps for s, t in per_stage.items()}
    ms_per_step = wall * 1e3 / args.steps

    flops = kernel_flops(B, H, n, d, causal)
    nbytes = kernel_bytes(B, H, n, d)
    step_flops = (4 + 10) * d * B * H * visible_pairs(n, n, causal)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    for s in stages:
        t = per_stage[s] * 1e-3
        kernels[s] = {
            "ms": round(per_stage[s], 4),
            "tflops": round(flops[s] / t / 1e12, 2),
            "gbs": round(nbytes[s] / t / 1e9, 1),
        }
    dominant = max(stages, key=lambda s: per_stage[s])
    dom_t = per_stage[dominant] * 1e-3
    achieved = flops[dominant] / dom_t / 1e12
    traffic = load_traffic(dominant, f"c3_fwdbwd_{'causal' if causal else 'noncausal'}_b{B}h{H}n{n}d{d}")
    fwd_lit = 4 * B * H * n * n * d / (per_stage["fwd"] * 1e-3) / 1e12
    # Each pass counted two ways: literal 4*B*H*n^2*d (the metric's formula,
    # all n^2 pairs, one product pair per pass), and algorithmic (visible
    # pairs; forward 2 products, backward 5, 2*d FLOP per pair each).
    t_fwd = per_stage["fwd"] * 1e-3
    t_bwd = (per_stage["bwd_preprocess"] + per_stage["bwd_dkdv"] + per_stage["bwd_dq"]) * 1e-3
    lit = 4 * B * H * n * n * d
    pairs = B * H * visible_pairs(n, n, causal)
    flop_report = {
        "fwd": {"ms": round(t_fwd * 1e3, 4), "flop_literal": lit, "flop_algorithmic": 4 * d * pairs,
                "tflops_literal": round(lit / t_fwd / 1e12, 2),
                "tflops_algorithmic": round(4 * d * pairs / t_fwd / 1e12, 2)},
        "bwd": {"ms": round(t_bwd * 1e3, 4), "flop_literal": lit, "flop_algorithmic": 10 * d * pairs,
                "tflops_literal": round(lit / t_bwd / 1e12, 2),
                "tflops_algorithmic": round(10 * d * pairs / t_bwd / 1e12, 2)},
        "step": {"flop_literal": 2 * lit, "flop_algorithmic": step_flops,
                 "tflops_literal": round(2 * lit / (ms_per_step * 1e-3) / 1e12, 2),
                 "tflops_algorithmic": round(value, 2)},
    }
    fwd_pct = 100 * flops["fwd"] / (per_stage["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v, dO; no dataset)",
        "config": {"workload": w.name, "B": B, "H": H, "n": n, "d": d, "causal": causal,
                   "scale": w.scale, "step": "fa_forward + fa_backward stages"},
        "fwd_tflops_literal": round(fwd_lit, 2),
        "fwd_pct_bf16_peak": round(fwd_pct, 2),
        "sclk_mhz_mean_fwd": sclk,
        "fwd_pct_bf16_peak_at_sclk": round(fwd_pct * PEAK_SCLK_MHZ / sclk, 2) if sclk else None,
        "kernels": kernels,
        "flops": flop_report,
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] in ("summarize-trace", "record-traffic", "summarize-counters"):
        sys.exit(profile_main(sys.argv[1:]))
    sys.exit(main())
