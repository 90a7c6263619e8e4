"""Host logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic byte and pair
counts the roofline divides by, the lookup of the committed HBM counter profile, and the
summaries of rocprofv3's CSV output that the profiles under profiles/ are made from."""
import os
import subprocess
import sys

import pytest

import bench
from sinks_ts_mha_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_algorithmic_bytes_full_layer():
    # q and out: 8192 tokens x 64 heads x 64 bf16 each; k and v: 8192 x 8 x 64 bf16
    # each; 64 fp32 sinks; 5 int32 cu_seqlens
    wl = workloads.get("gptoss_full_4x2048")
    expect = 2 * 8192 * 64 * 64 * 2 + 2 * 8192 * 8 * 64 * 2 + 64 * 4 + 5 * 4
    assert bench.algorithmic_bytes(wl) == expect == 150995220


def test_algorithmic_bytes_head_dim_128():
    wl = workloads.get("d128_full_4x2048")
    expect = 2 * 8192 * 64 * 128 * 2 + 2 * 8192 * 8 * 128 * 2 + 64 * 4 + 5 * 4
    assert bench.algorithmic_bytes(wl) == expect


def test_cache_visible_pairs_brute_force():
    # new rows at the end of each sequence's keys, counted key by key
    wl = workloads.CacheWorkload("t", (2, 3, 1), (5, 3, 70), 16, 2, 16, window=0)
    got = bench.cache_visible_pairs(wl)
    ref = sum(1 for q, L in zip(wl.q_lens, wl.k_lens) for i in range(q) for j in range(L)
              if j <= L - q + i)
    assert got == ref
    ww = workloads.CacheWorkload("t", (2, 3, 1), (5, 3, 70), 16, 2, 16, window=2)
    got = bench.cache_visible_pairs(ww)
    ref = sum(1 for q, L in zip(ww.q_lens, ww.k_lens) for i in range(q) for j in range(L)
              if 0 <= (L - q + i) - j < 2)
    assert got == ref


def test_read_traffic_uses_only_a_matching_profile(monkeypatch):
    wl = workloads.get("gptoss_full_4x2048")
    t = bench.read_traffic("gptoss_full_4x2048")
    if t is not None:  # the committed profile matches the kernel source
        assert 0.99 < t / bench.algorithmic_bytes(wl) < 1.5
    # a profile taken for other kernel code is ignored
    monkeypatch.setattr(bench, "source_sha", lambda head_dim=64: "0" * 64)
    assert bench.read_traffic("gptoss_full_4x2048") is None
    # and so is a workload without a profile
    assert bench.read_traffic("no_such_workload") is None


def test_trace_summary_takes_the_last_prefill_dispatches(tmp_path, capsys):
    d = tmp_path / "run"
    d.mkdir()
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for dur in (900, 100, 200, 300):  # a warm-up dispatch, then the timed ones
        rows.append(f"\"void tsmha::prefill_fwd_d64<8, false, false>(tsmha::KParams)\",{t},{t + dur}")
        t += 1000
    rows.append(f"__amd_rocclr_copyBuffer,{t},{t + 50}")
    (d / "x_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.trace_summary(str(tmp_path), 3)
    out = capsys.readouterr().out
    assert "timed region (last 3 prefill dispatches): avg_ns 200.0 min_ns 100 max_ns 300" in out


def test_counter_summary_sums_instances_per_dispatch(tmp_path, capsys):
    rows = ["Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value"]
    for disp, vals in ((1, (10, 20)), (2, (30, 40))):  # two counter instances per dispatch
        for v in vals:
            rows.append(f"{disp},k,256,FETCH_SIZE,{v}")
    (tmp_path / "a_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.counter_summary(str(tmp_path))
    line = [l for l in capsys.readouterr().out.splitlines() if "FETCH_SIZE" in l][0]
    parts = line.split()
    assert parts[-2] == "2" and float(parts[-1]) == pytest.approx(50.0)


def test_trace_summary_phases(tmp_path, capsys):
    """Phases split one kernel's dispatches at a grid change or a pause over 20 ms; another
    kernel's dispatches in between (a merge kernel after each split) do not split them."""
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X"]
    t = 0
    for grid, durs in ((512, (500, 100, 100)), (512, (700, 300, 300)), (256, (50, 40))):
        t += 30_000_000  # a pause between workloads
        for dur in durs:
            rows.append(f"split,{t},{t + dur},{grid}")
            rows.append(f"merge,{t + dur},{t + dur + 5},64")
            t += 1000
    (tmp_path / "y_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.trace_summary(str(tmp_path), 2)
    lines = [l.split() for l in capsys.readouterr().out.splitlines() if l[:3].strip().isdigit()]
    split = [(int(l[2]), int(l[3]), float(l[4])) for l in lines if l[1] == "split"]
    assert split == [(512, 3, 100.0), (512, 3, 300.0), (256, 2, 45.0)]
    assert sum(1 for l in lines if l[1] == "merge") == 3
