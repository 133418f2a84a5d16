"""CPU tests of bench.py's host logic: the algorithmic FLOP and byte counts
that the roofline figures divide by, the kernel-name classification, and the
profiler-summary code that turns rocprofv3 CSV files into the records under
profiles/ (run here on small synthetic CSV files in a scratch tree, so the
committed records are never touched)."""
import csv
import json
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ------------------------------------------------------------ counts

@pytest.mark.parametrize("n_q,n_k", [(1, 1), (5, 5), (7, 3), (3, 7), (16, 33), (40, 17)])
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_brute_force(n_q, n_k, causal):
    # the mask the kernels and the oracle apply at offset 0: row i sees key j iff j <= i
    want = sum(1 for i in range(n_q) for j in range(n_k) if not causal or j <= i)
    assert bench.visible_pairs(n_q, n_k, causal) == want


def test_step_flops_add_up_to_fourteen_d_per_visible_pair():
    # forward 4d (two products), dK/dV 8d (S, dP, dV, dK), dQ 2d: the
    # 14·d per visible pair that the oracle CPU figure uses too
    for causal in (False, True):
        f = bench.kernel_flops(1, 32, 4096, 128, causal)
        pairs = 32 * bench.visible_pairs(4096, 4096, causal)
        assert f["fwd"] + f["bwd_dkdv"] + f["bwd_dq"] == 14 * 128 * pairs
    # the metric's 4·B·H·n²·d for the non-causal forward, and a causal forward
    # of n(n+1)/2 pairs per head
    assert bench.kernel_flops(2, 3, 10, 8, False)["fwd"] == 4 * 2 * 3 * 10 ** 2 * 8
    assert bench.kernel_flops(2, 3, 10, 8, True)["fwd"] == 4 * 2 * 3 * 55 * 8


def test_kernel_bytes_at_n4096_d128():
    mib = 1 << 20
    b = bench.kernel_bytes(1, 32, 4096, 128)
    # one bf16 (32, 4096, 128) tensor is 32 MiB; one fp32 row vector 512 KiB
    assert b["fwd"] == 4 * 32 * mib + mib // 2              # q k v read, o written, lse written
    assert b["bwd_dkdv"] == 6 * 32 * mib + 2 * (mib // 2)   # q k v dO read, dk dv written
    assert b["bwd_dq"] == 5 * 32 * mib + 2 * (mib // 2)
    assert b["bwd_preprocess"] == 2 * 32 * mib + 3 * (mib // 2)


def test_decode_bytes_are_the_cache_plus_the_queries():
    # B=4, 8 K/V heads, 32768 keys, d=128, bf16: K and V are 512 MiB together
    full = bench.decode_bytes(4, 64, 8, 1, 32768, 128)
    none = bench.decode_bytes(4, 64, 8, 1, 0, 128)
    assert full - none == 512 << 20
    assert none == 4 * 64 * (2 * 128 * 2 + 4)   # q read and o written (bf16), lse written (fp32)


# ------------------------------------------------------------ kernel names

def _library_kernels():
    names = set()
    csrc = os.path.join(ROOT, "exact_attention_05_amd", "csrc")
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(csrc, f)).read()
            names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", text, re.S))
    return sorted(names)


def test_every_library_kernel_has_a_stage():
    names = _library_kernels()
    assert len(names) >= 10, names
    for name in names:
        assert bench.stage_of(f"void fa::(anonymous namespace)::{name}<128, false>(fa::Args)") is not None, name


@pytest.mark.parametrize("name,stage", [
    ("void fa::fwdk::fwd_bf16_pp_kernel<128, false, false>(fa::FwdArgs, int)", "fwd"),
    ("void fa::fwdk::fwd_f32_split16_kernel<64, true>(fa::FwdArgs, int)", "fwd"),
    ("_ZN2fa12_GLOBAL__N_121bwd_preprocess_kernelILi128EDF16bEEvPKT0_S4_PKfPfS7_l", "bwd_preprocess"),
    ("void fa::(anonymous namespace)::bwd_dkdv_bf16_kernel<128, false, 0, 4>(fa::BwdArgs, int)", "bwd_dkdv"),
    ("void fa::(anonymous namespace)::bwd_dq_bf16_pp_kernel<128, false>(fa::BwdArgs, int)", "bwd_dq"),
    ("void fa::(anonymous namespace)::bwd_reduce_slices_kernel<float>(fa::BwdArgs, long long)", "bwd_reduce"),
    ("void fa::(anonymous namespace)::decode_bf16_kernel<128, true, 4>(fa::DecArgs)", "decode"),
    ("_ZN2fa12_GLOBAL__N_116lse_merge_kernelILi128EfDF16bEEvNS_9MergeArgsE", "lse_merge"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::BinaryFunctor<float, float, float, "
     "at::native::binary_internal::MulFunctor<float> >, std::array<char*, 3ul> >(int, "
     "at::native::BinaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> >, "
     "std::array<char*, 3ul>)", None),
])
def test_stage_of(name, stage):
    assert bench.stage_of(name) == stage


# ------------------------------------------------------------ profiler summaries

FWD = "void fa::fwdk::fwd_bf16_pp_kernel<128, false, false>(fa::FwdArgs, int)"
DQ = "void fa::(anonymous namespace)::bwd_dq_bf16_pp_kernel<128, false>(fa::BwdArgs, int)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, std::array<char*, 1ul> >"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>, std::array<char*, 3ul> >"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


@pytest.fixture()
def tree(tmp_path, monkeypatch):
    """A scratch repository root with stand-in kernel sources and an empty profiles/."""
    csrc = tmp_path / "exact_attention_05_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "common.hpp"):
        (csrc / f).write_text(f"// {f}\n")
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "fa.h").write_text("// fa.h\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _counter_rows(counter, values):
    return [{"Dispatch_Id": str(i), "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": str(v)}
            for i, k, v in values]


def test_traffic_record_round_trip(tree):
    kib = bench.COPY_KIB
    # rows out of dispatch order: the record must take each kernel's last dispatch
    fetch = _counter_rows("FETCH_SIZE", [(5, FWD, 50), (1, FILL, 3), (2, COPY, kib // 2), (3, FWD, 100),
                                         (4, DQ, 70)])
    write = _counter_rows("WRITE_SIZE", [(1, FILL, kib), (2, COPY, kib), (3, FWD, 40), (4, DQ, 10),
                                         (5, FWD, 30)])
    _write_csv(str(tree / "f" / "host" / "1_counter_collection.csv"), fetch)
    _write_csv(str(tree / "w" / "host" / "1_counter_collection.csv"), write)
    md = bench.record_traffic(str(tree / "f"), str(tree / "w"), "wl", ["cmd one", "cmd two"])
    text = open(md).read()
    assert "cmd one" in text and "fetch x2.000, write x1.000" in text
    rec = json.load(open(tree / "profiles" / "traffic_fwd.json"))
    # the copy read half its true bytes, so fetch counts are doubled
    assert rec["bytes_per_launch"] == (50 * 2 + 30) * 1024
    assert rec["fetch_kib"] == 50 and rec["write_kib"] == 30 and rec["workload"] == "wl"
    assert bench.load_traffic("fwd", "wl") == (50 * 2 + 30) * 1024
    assert bench.load_traffic("bwd_dq", "wl") == (70 * 2 + 10) * 1024
    # no record for a kernel that did not run, nor for another workload
    assert bench.load_traffic("bwd_dkdv", "wl") is None
    assert bench.load_traffic("fwd", "other") is None
    # a change to any header the kernel can include voids the record
    (tree / "exact_attention_05_amd" / "csrc" / "common.hpp").write_text("// changed\n")
    assert bench.load_traffic("fwd", "wl") is None


def test_source_digest_covers_the_kernel_its_headers_and_the_abi_header(tree):
    d0 = bench.kernel_source_digest("fwd")
    assert bench.kernel_source_digest("bwd_dq") != d0
    assert bench.kernel_source_digest("bwd_dq") == bench.kernel_source_digest("bwd_dkdv")
    (tree / "exact_attention_05_amd" / "csrc" / "fa_bwd.hip").write_text("// other\n")
    assert bench.kernel_source_digest("fwd") == d0
    (tree / "include" / "fa.h").write_text("// other\n")
    assert bench.kernel_source_digest("fwd") != d0


def test_trace_summary_means_the_last_timed_calls(tree):
    us = 1000
    stats = [{"Name": FWD, "Calls": "4", "TotalDurationNs": str(100 * us), "AverageNs": str(25 * us),
              "Percentage": "80.0", "MinNs": str(10 * us), "MaxNs": str(40 * us)},
             {"Name": COPY, "Calls": "1", "TotalDurationNs": str(25 * us), "AverageNs": str(25 * us),
              "Percentage": "20.0", "MinNs": str(25 * us), "MaxNs": str(25 * us)}]
    # dispatches of 10, 20, 30, 40 us, written out of time order
    trace = [{"Kernel_Name": FWD, "Start_Timestamp": str(t), "End_Timestamp": str(t + dur * us)}
             for t, dur in ((3000000, 40), (1000000, 20), (0, 10), (2000000, 30))]
    trace.append({"Kernel_Name": COPY, "Start_Timestamp": "5000000", "End_Timestamp": str(5000000 + 25 * us)})
    _write_csv(str(tree / "t" / "host" / "1_kernel_stats.csv"), stats)
    _write_csv(str(tree / "t" / "host" / "1_kernel_trace.csv"), trace)
    path = bench.summarize_trace(str(tree / "t"), "wl", ["the command"], 2, "a note")
    lines = open(path).read().splitlines()
    fwd = [ln for ln in lines if "fwd_bf16_pp_kernel" in ln]
    assert len(fwd) == 1 and "| 25.0 | 10.0 | 40.0 | 80.0% | 35.0 (last 2) |" in fwd[0]
    assert lines.index(fwd[0]) < [i for i, ln in enumerate(lines) if "MulFunctor" in ln][0]


def test_counter_summary_utilisation(tree):
    # pass one: products and busy cycles; pass two: the clock counter
    a = [{"Dispatch_Id": "1", "Kernel_Name": FWD, "Counter_Name": c, "Counter_Value": str(v)}
         for c, v in (("SQ_INSTS_MFMA", 1000), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500),
                      ("SQ_INSTS_VALU", 2500))]
    b = [{"Dispatch_Id": "1", "Kernel_Name": FWD, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": str(8 * 1000)},
         {"Dispatch_Id": "2", "Kernel_Name": COPY, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": "8"}]
    _write_csv(str(tree / "p1" / "host" / "1_counter_collection.csv"), a)
    _write_csv(str(tree / "p2" / "host" / "1_counter_collection.csv"), b)
    path = bench.summarize_counters([str(tree / "p1"), str(tree / "p2")], "wl", ["c1", "c2"])
    row = [ln for ln in open(path).read().splitlines() if ln.startswith("| fwd | 1000 |")]
    assert len(row) == 1
    assert "| 1000 | 500 | 1000 | 50.0 % | 2.50 |" in row[0]
    assert "MulFunctor" not in open(path).read()   # kernels outside the library are left out


# ------------------------------------------------------------ command line

def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2


def test_unknown_profile_command_prints_its_usage():
    with pytest.raises(SystemExit) as e:
        bench.profile_main(["nonsense"])
    assert "record-traffic" in str(e.value)
