"""Benchmark: prefill attention TFLOP/s (unmasked pairs) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --sweep            # the chart family: one JSON line per point
    python bench.py --decode           # decode against a paged KV cache: one line per workload
    python bench.py --prefill-kvcache  # new rows against a paged KV cache: one line per workload

One step is one ts_mha_prefill call over the whole workload: every stage of the
operation (tile walk, QK^T, mask, online softmax with sink, PV, epilogue) runs
inside that single kernel launch.  Inputs are seeded synthetic tensors already
resident in device memory when the timed region starts.  Warm-up runs at least
--warmup launches and at least --warmup-seconds (default 1 s) of them: under a
sudden load the GPU's clocks take tens of milliseconds to settle, and launches
in that ramp run up to 25% slower than in steady state.

    python bench.py --trace-summary DIR --steps K   # durations from a rocprofv3 kernel trace

Metric: FLOP = 4 * head_dim * n_q_heads * (visible query-key pairs per head),
i.e. 2*head_dim flops for q.k and 2*head_dim for the weighted sum of v, counted
only on unmasked pairs.  Printed as one JSON line with a `roofline` object (the
kernel's average duration from HIP events on the launch stream against the
bf16 dense MFMA peak) and a `cpu_baseline` object (the fp64 oracle timed on
this host's cores on a bounded row sample of the same workload).  The line also
carries:
  per_launch        median / min / max of launches timed one by one, each between
                    its own event pair (the pairs add their own gaps; the mean of
                    the back-to-back launches above stays the figure);
  roofline_valu     the vector ALU's roof: every visible score costs the softmax one
                    v_mul_f32, one v_exp_f32 and half a v_cvt_pk_bf16_f32, and the
                    microbenchmark (--ubench) gives the chip's rate of that mix at the
                    kernel's occupancy; achieved = n_q_heads * visible pairs / kernel time;
  mfma_sustained_tflops  the microbenchmark's back-to-back bf16 32x32x16 MFMA rate;
  device            CU count and clocks from hipDeviceGetAttribute;
  roofline_hbm, roofline_hbm_cold  (windowed workloads) algorithmic bytes over the
                    kernel time, warm (back-to-back launches on resident inputs) and
                    cold (the median of --cold-launches launches timed one by one,
                    each after writing --flush-mib MiB of scratch, which leaves no
                    line of the workload in the L2s or the last-level cache).

    python bench.py --ubench   # issue rates of exp2, multiply, bf16 pack, the softmax
                               # mix and the MFMA, and the device's CU count and clocks

--decode times ts_mha_decode_with_kvcache on the paged-cache workloads: one step
is one call (the split kernel and, for long sequences, the merge kernel), and the
figure is algorithmic HBM bytes per second (every visible cached key and value
read once, q read, out written).  `value` uses the wall time of eager calls
(host overhead included); `gpu_avg_us` and `frac_hbm` (against the 8 TB/s roof)
use the same calls replayed from one captured HIP graph.

--sweep times the chart family (full causal, 64/8 heads, head_dim 64, batch x
seq_len): `kernel_avg_us` and `frac` from the eager launches' event pair (on the
smallest points the host's per-call overhead exceeds the kernel and shows up as
gaps), `graph_avg_us` and `frac_graph` from the same launches replayed from one
captured HIP graph (no host call per launch, but the graph's own gap between
nodes, a few microseconds).  A kernel trace gives the kernel's own duration.

--prefill-kvcache times ts_mha_prefill_with_kvcache (chunked prefill: new rows at
the end of each sequence's cached keys) and reports TFLOP/s over the visible
(query, key) pairs, as the main metric does, against the bf16 MFMA peak.

Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E bandwidth
KERNEL_SOURCES = {64: os.path.join(ROOT, "sinks_ts_mha_amd", "csrc", "prefill_fwd.hip"),
                  128: os.path.join(ROOT, "sinks_ts_mha_amd", "csrc", "prefill_fwd_narrow.hip")}
METRIC = "prefill attention TFLOP/s (unmasked pairs) and % of MI355X bf16 MFMA peak"


def source_sha(head_dim: int = 64) -> str:
    """Hash of the prefill kernel source's code for head_dim: comments and whitespace do not count."""
    text = open(KERNEL_SOURCES[head_dim]).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it is for this kernel source."""
    path = os.path.join(ROOT, "profiles", f"pmc_prefill_fwd_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^([A-Za-z0-9_]+):\s*(.+?)\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    from sinks_ts_mha_amd import workloads
    if kv.get("source_sha256") != source_sha(workloads.get(workload).head_dim):
        return None
    try:
        fetch = float(kv["FETCH_SIZE_KiB_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
        write = float(kv["WRITE_SIZE_KiB_per_dispatch"]) * 1024 * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def algorithmic_bytes(wl) -> int:
    T, D = wl.total_tokens, wl.head_dim
    return T * (2 * wl.n_q_heads * D + 2 * wl.n_kv_heads * D) * 2 + 4 * wl.n_q_heads + \
        4 * (len(wl.seqlens) + 1)


def decode_algorithmic_bytes(wl) -> int:
    """Bytes a decode step must move: visible K and V rows, q, out, seqlens, page ids, sinks."""
    D = wl.head_dim
    vis = [min(L, wl.window) if wl.window > 0 else L for L in wl.k_lens]
    pages = sum(-(-v // wl.page_size) for v in vis)
    return (sum(vis) * wl.n_kv_heads * D * 2 * 2 + 2 * wl.n_seqs * wl.n_q_heads * D * 2
            + 4 * wl.n_seqs + 4 * pages + 4 * wl.n_q_heads)


def cache_visible_pairs(wl) -> int:
    """Visible (query, key) pairs per head of new rows at the end of each sequence's keys."""
    total = 0
    for q, L in zip(wl.q_lens, wl.k_lens):
        off = L - q
        for i in range(q):
            n = off + i + 1
            total += min(n, wl.window) if wl.window > 0 else n
    return total


def cpu_baseline(wl, inp, target_s: float):
    """Time the fp64 oracle on a strided row sample sized for about target_s seconds."""
    import numpy as np

    from oracle import oracle
    from sinks_ts_mha_amd.workloads import bf16_bits

    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    if not os.path.exists(os.path.join(ROOT, "oracle", "libts_oracle.so")):
        oracle.build()
    args = (bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]),
            inp["sinks"].numpy() if inp["sinks"] is not None else None,
            inp["cu_seqlens"].numpy(), inp["window"], inp["softmax_scale"])
    cu = inp["cu_seqlens"].numpy().astype(np.int64)
    W = inp["window"]
    pos_all, tok_all = [], []
    for b in range(len(cu) - 1):
        i = np.arange(cu[b + 1] - cu[b])
        pos_all.append(i)
        tok_all.append(cu[b] + i)
    pos_all = np.concatenate(pos_all)
    tok_all = np.concatenate(tok_all)
    keys = np.minimum(pos_all + 1, W) if W > 0 else pos_all + 1
    hq, D = wl.n_q_heads, wl.head_dim

    def run(stride):
        sel = np.arange(0, tok_all.size, stride)
        rows = np.repeat(tok_all[sel], hq)
        heads = np.tile(np.arange(hq, dtype=np.int32), sel.size)
        t0 = time.perf_counter()
        oracle.prefill_rows(*args, rows=rows, heads=heads)
        dt = time.perf_counter() - t0
        return dt, float(keys[sel].sum()) * hq * 4 * D, sel.size

    # probe with a thin sample, then size the real one for the target time
    dt, flops, _ = run(max(1, tok_all.size // 64))
    rate = flops / max(dt, 1e-6)
    total_flops = float(keys.sum()) * hq * 4 * D
    stride = max(1, int(round(total_flops / max(rate * target_s, 1.0))))
    dt, flops, n = run(stride)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"every packed token ({n})" if stride == 1 else
                       f"one packed token in {stride} ({n} of {tok_all.size})") + f", all {hq} q heads, "
                      f"fp64 oracle rows; {dt:.1f} s wall"}


UBENCH_OPS = {"exp2": 0, "mul": 1, "cvt_pk_bf16": 2, "softmax_score": 3, "mfma_32x32x16_bf16": 4}


def ubench_lib():
    """The microbenchmark library (sinks_ts_mha_amd/libts_ubench.so), built beside libts_mha.so."""
    import ctypes
    path = os.path.join(ROOT, "sinks_ts_mha_amd", "libts_ubench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with `python -m sinks_ts_mha_amd.build`")
    L = ctypes.CDLL(path)
    ip = ctypes.POINTER(ctypes.c_int)
    L.ts_ubench_device_info.argtypes = [ip, ip, ip, ip]
    L.ts_ubench_device_info.restype = ctypes.c_int
    L.ts_ubench_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.ts_ubench_valu.restype = ctypes.c_int
    return L


def device_info() -> dict:
    """CU count and clocks of the current device, from hipDeviceGetAttribute."""
    import ctypes
    v = [ctypes.c_int(0) for _ in range(4)]
    if ubench_lib().ts_ubench_device_info(*[ctypes.byref(x) for x in v]) != 0:
        raise RuntimeError("hipDeviceGetAttribute failed")
    return {"cus": v[0].value, "clock_mhz": v[1].value / 1000.0, "mem_clock_mhz": v[2].value / 1000.0,
            "mem_bus_bits": v[3].value}


def ubench_rates(names=None, target_ms: float = 8.0) -> dict:
    """Issue rates of the microbenchmark kernels on every compute unit at two waves per SIMD
    (two work-groups of four waves per CU): each lane runs 16 independent chains of the
    instruction kind per loop trip.  Per kind: wave-level instructions per second, the SIMD
    cycles one instruction takes at the device's reported clock, and for the softmax kind
    the scores per second (one v_mul_f32, one v_exp_f32 and half a v_cvt_pk_bf16_f32 each),
    for the MFMA kind the dense bf16 TFLOP/s (32768 flops per instruction)."""
    import torch
    L = ubench_lib()
    info = device_info()
    groups = 2 * info["cus"]
    out = torch.empty(groups * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name in (names or UBENCH_OPS):
        op = UBENCH_OPS[name]

        def launch(iters):
            if L.ts_ubench_valu(op, groups, iters, out.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError(f"microbenchmark {name} failed to launch")

        iters = 256
        for _ in range(8):  # size the launch for about target_ms
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(iters)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if ms >= target_ms / 2:
                break
            iters *= 2
        times = []
        for _ in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(iters)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(times)[len(times) // 2]
        insts = groups * 4 * iters * 16
        r = {"wave_instructions_per_s": insts / t,
             "simd_cycles_per_instruction": info["cus"] * 4 * info["clock_mhz"] * 1e6 * t / insts,
             "median_launch_ms": round(t * 1e3, 3)}
        if name == "softmax_score":
            r["scores_per_s"] = insts * 64 / t
        if name == "mfma_32x32x16_bf16":
            r["tflops"] = insts * 32768 / t / 1e12
        res[name] = r
    return res


def trace_summary(root: str, last: int):
    """Per-kernel durations from rocprofv3's kernel_trace.csv files under root: every dispatch,
    and the last `last` prefill dispatches (the timed region of a bench.py run)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                grid = r.get("Grid_Size_X") or r.get("Grid_Size") or "0"
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                             r["Kernel_Name"], int(grid)))
    rows.sort()
    names = sorted({n for _, _, n, _ in rows})
    print(f"{'kernel':70s} {'calls':>6s} {'avg_ns':>12s} {'min_ns':>10s} {'max_ns':>10s}")
    for n in names:
        d = [x for _, x, k, _ in rows if k == n]
        print(f"{n[:70]:70s} {len(d):6d} {sum(d) / len(d):12.1f} {min(d):10d} {max(d):10d}")
    d = [x for _, x, k, _ in rows if "prefill_fwd" in k][-last:]
    if d:
        print(f"timed region (last {len(d)} prefill dispatches): avg_ns {sum(d) / len(d):.1f} "
              f"min_ns {min(d)} max_ns {max(d)}")
    # Phases: the dispatches of one kernel with one grid size in a row (other kernels' dispatches
    # in between do not break a phase; a grid change or a pause of over 20 ms does), i.e. the
    # warm-up and timed launches of one workload; the average is over the phase's last `last`.
    print(f"phases (per kernel: runs of one grid size, split at pauses over 20 ms; avg and min of the last "
          f"{last} dispatches of each):")
    print(f"{'#':>3s} {'kernel':60s} {'grid':>9s} {'calls':>6s} {'avg_ns':>12s} {'min_ns':>10s}")
    phases = []
    for n in names:
        cur = None
        for t, x, k, g in rows:
            if k != n:
                continue
            if cur is None or g != cur["grid"] or t - cur["end"] > 20_000_000:
                cur = {"name": n, "grid": g, "start": t, "end": t + x, "d": []}
                phases.append(cur)
            cur["d"].append(x)
            cur["end"] = t + x
    for i, ph in enumerate(sorted(phases, key=lambda p: p["start"])):
        d = ph["d"][-last:]
        print(f"{i:3d} {ph['name'][:60]:60s} {ph['grid']:9d} {len(ph['d']):6d} {sum(d) / len(d):12.1f} {min(d):10d}")


def counter_summary(root: str):
    """Average value per dispatch of each counter, per kernel and grid size, in rocprofv3's
    counter_collection.csv files under root."""
    import csv
    import glob
    acc = {}
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"])
                d = acc.setdefault(key, {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    print(f"{'kernel':64s} {'grid':>8s} {'counter':12s} {'dispatches':>10s} {'avg_per_dispatch':>17s}")
    for (k, g, c), d in sorted(acc.items()):
        print(f"{k[:64]:64s} {g:8d} {c:12s} {len(d):10d} {sum(d.values()) / len(d):17.3f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up until this much time has passed as well (the GPU's "
                         "clocks take tens of milliseconds of load to reach their steady state)")
    ap.add_argument("--counter-summary", default=None, metavar="DIR",
                    help="average per dispatch of each counter of a rocprofv3 --pmc run under DIR, and exit")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="summarise the prefill dispatches of a rocprofv3 kernel trace under DIR "
                         "(the last --steps of them: the timed region) and exit")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every chart point (sequence length x batch, full causal) instead")
    ap.add_argument("--decode", action="store_true",
                    help="time decode against a paged KV cache on its workloads instead")
    ap.add_argument("--prefill-kvcache", action="store_true",
                    help="time prefill of new rows against a paged KV cache instead")
    ap.add_argument("--ubench", action="store_true",
                    help="print the vector-ALU and MFMA issue rates of the microbenchmarks and the "
                         "device's CU count and clocks instead")
    ap.add_argument("--cold-launches", type=int, default=50,
                    help="windowed workloads: launches timed one by one after writing --flush-mib "
                         "of scratch memory each (the cold-cache figure)")
    ap.add_argument("--flush-mib", type=int, default=512)
    ap.add_argument("--per-launch", type=int, default=200,
                    help="launches timed one by one (own event pair each) for the median and minimum")
    a = ap.parse_args()
    if a.trace_summary:
        trace_summary(a.trace_summary, a.steps)
        return
    if a.counter_summary:
        counter_summary(a.counter_summary)
        return
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              "(the operation shards by KV-head group or by sequence with no exchange, "
              "so one GPU's throughput is the figure measured here).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sinks_ts_mha_amd as tm
    from sinks_ts_mha_amd import workloads

    if a.ubench:
        print(json.dumps({"device": device_info(), "ubench": ubench_rates()}), flush=True)
        return

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    warm_counts = {}
    per_launch = {}
    cold_launch = {}

    def warm(fn) -> int:
        """At least --warmup launches and at least --warmup-seconds of them; returns the count."""
        n, t = 0, time.perf_counter()
        while n < a.warmup or time.perf_counter() - t < a.warmup_seconds:
            for _ in range(25):
                fn()
            n += 25
            torch.cuda.synchronize()
        return n

    def timed(wl, steps, warmup, copy_calibration=False, graph_replay=False):
        """Resident inputs, W warm-up launches, then K launches timed on the host clock and by
        one pair of HIP events on the launch stream: (inputs, ms per step, kernel avg ms,
        graph-replay avg ms or None)."""
        inp = workloads.make_inputs(wl)
        q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
        sinks = inp["sinks"].to(dev) if inp["sinks"] is not None else None
        cu = inp["cu_seqlens"].to(dev)
        out = torch.empty_like(q)

        def step():
            tm.ts_mha_prefill(q, k, v, sinks, cu, window=wl.window, softmax_scale=wl.softmax_scale,
                              out=out, max_seqlen=wl.max_seqlen, stream=stream)

        if copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        warm_counts[wl.name] = warm(step)
        # One event pair on the launch stream around the K back-to-back launches:
        # the GPU-side span divided by K is the kernel's average launch duration
        # (events between launches would add their own dispatch gaps).
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # The same launches timed one by one, each between its own event pair, for the
        # median and minimum (the pairs add their own gaps, so the mean above stays the
        # figure); with cold=True each is preceded by writing flush_mib of scratch, which
        # leaves neither the L2s nor the last-level cache holding the workload's lines.
        def one_by_one(n, cold):
            flush = torch.empty(a.flush_mib << 20, dtype=torch.uint8, device=dev) if cold else None
            pairs = []
            for i in range(n):
                if cold:
                    flush.fill_(i & 0xff)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step()
                e1.record(stream)
                pairs.append((e0, e1))
            torch.cuda.synchronize()
            ms = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
            del flush
            return {"median_us": round(ms[len(ms) // 2] * 1e3, 2), "min_us": round(ms[0] * 1e3, 2),
                    "max_us": round(ms[-1] * 1e3, 2), "launches": n}
        per_launch[wl.name] = one_by_one(min(steps, a.per_launch), False) if a.per_launch > 0 else None
        if wl.window > 0 and a.cold_launches > 0:
            cold_launch[wl.name] = one_by_one(a.cold_launches, True)
        ms_graph = None
        if graph_replay:
            # The same K launches captured in one HIP graph, replayed between one pair of
            # events on the replay stream: GPU time without the host's per-call overhead
            # (which on the smallest workloads exceeds the kernel's own duration), with the
            # graph's own gap between nodes instead.
            graph = torch.cuda.CUDAGraph()
            gs = torch.cuda.Stream()
            gs.wait_stream(stream)
            with torch.cuda.stream(gs):
                with torch.cuda.graph(graph, stream=gs):
                    for _ in range(steps):
                        tm.ts_mha_prefill(q, k, v, sinks, cu, window=wl.window,
                                          softmax_scale=wl.softmax_scale, out=out,
                                          max_seqlen=wl.max_seqlen)
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(gs):
                graph.replay()
                torch.cuda.synchronize()
                g0.record(gs)
                graph.replay()
                g1.record(gs)
            torch.cuda.synchronize()
            ms_graph = g0.elapsed_time(g1) / steps
            del graph
        del q, k, v, sinks, cu, out
        return inp, wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps, ms_graph

    if a.prefill_kvcache:
        for name, wl in workloads.PREFILL_KV_WORKLOADS.items():
            inp = workloads.make_cache_inputs(wl)
            q, kc, vc = inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev)
            sinks = inp["sinks"].to(dev) if inp["sinks"] is not None else None
            cuq, lens = inp["cu_seqlens_q"].to(dev), inp["seqlens_k"].to(dev)
            table = inp["block_table"].to(dev)
            out = torch.empty_like(q)

            def pstep():
                tm.ts_mha_prefill_with_kvcache(q, kc, vc, sinks, cuq, lens, table, window=wl.window,
                                               softmax_scale=wl.softmax_scale, out=out,
                                               max_seqlen_q=wl.max_seqlen_q,
                                               max_seqlen_k=wl.max_seqlen_k, stream=stream)

            n_warm = warm(pstep)
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev0.record(stream)
            for _ in range(a.steps):
                pstep()
            ev1.record(stream)
            torch.cuda.synchronize()
            ms_step = (time.perf_counter() - t0) * 1e3 / a.steps
            ms_gpu = ev0.elapsed_time(ev1) / a.steps
            flops = 4 * wl.head_dim * wl.n_q_heads * cache_visible_pairs(wl)
            print(json.dumps({"prefill_kvcache_point": name, "batch": wl.n_seqs,
                              "q_len": wl.max_seqlen_q, "k_len": wl.max_seqlen_k,
                              "window": wl.window, "page_size": wl.page_size,
                              "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                              "kernel_avg_us": round(ms_gpu * 1e3, 2),
                              "frac": round(flops / (ms_gpu * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "flops": flops, "steps": a.steps, "warmup": a.warmup,
                              "warmup_launches": n_warm}), flush=True)
            del q, kc, vc, sinks, cuq, lens, table, out
            torch.cuda.empty_cache()
        return

    if a.decode:
        for name, wl in workloads.DECODE_WORKLOADS.items():
            inp = workloads.make_cache_inputs(wl)
            q, kc, vc = inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev)
            sinks = inp["sinks"].to(dev) if inp["sinks"] is not None else None
            lens, table = inp["seqlens_k"].to(dev), inp["block_table"].to(dev)
            out = torch.empty_like(q)
            need = tm.ts_mha_decode_workspace_size(wl.n_seqs, wl.n_q_heads, wl.n_kv_heads,
                                                   wl.head_dim, wl.window, wl.max_seqlen_k)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

            def dstep():
                tm.ts_mha_decode_with_kvcache(q, kc, vc, sinks, lens, table, window=wl.window,
                                              softmax_scale=wl.softmax_scale, out=out,
                                              max_seqlen_k=wl.max_seqlen_k, workspace=ws,
                                              stream=stream)

            warm(dstep)
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(a.steps):
                dstep()
            torch.cuda.synchronize()
            ms_step = (time.perf_counter() - t0) * 1e3 / a.steps
            # GPU time without the host's launch overhead: the same K calls captured
            # in one HIP graph (the library records no memset), replayed between
            # one pair of events on the replay stream.
            graph = torch.cuda.CUDAGraph()
            gs = torch.cuda.Stream()
            gs.wait_stream(stream)
            with torch.cuda.stream(gs):
                with torch.cuda.graph(graph, stream=gs):
                    for _ in range(a.steps):
                        tm.ts_mha_decode_with_kvcache(q, kc, vc, sinks, lens, table,
                                                      window=wl.window,
                                                      softmax_scale=wl.softmax_scale, out=out,
                                                      max_seqlen_k=wl.max_seqlen_k, workspace=ws)
            # replay() launches on the current stream: the events go on that same stream
            with torch.cuda.stream(gs):
                graph.replay()
                torch.cuda.synchronize()
                ev0.record(gs)
                graph.replay()
                ev1.record(gs)
            torch.cuda.synchronize()
            ms_gpu = ev0.elapsed_time(ev1) / a.steps
            nbytes = decode_algorithmic_bytes(wl)
            print(json.dumps({"decode_point": name, "batch": wl.n_seqs, "k_len": wl.max_seqlen_k,
                              "window": wl.window, "page_size": wl.page_size,
                              "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
                              "host_us_per_step": round(ms_step * 1e3, 2),
                              "gpu_avg_us": round(ms_gpu * 1e3, 2),
                              "algorithmic_bytes": nbytes,
                              "frac_hbm": round(nbytes / (ms_gpu * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "workspace_bytes": need, "steps": a.steps, "warmup": a.warmup}),
                  flush=True)
            del graph
            del q, kc, vc, sinks, lens, table, out, ws
            torch.cuda.empty_cache()
        return

    if a.sweep:
        for wl in workloads.SWEEP.values():
            _, ms_step, ms_kernel, ms_graph = timed(wl, a.steps, a.warmup, graph_replay=True)
            flops = 4 * wl.head_dim * wl.n_q_heads * tm.ts_mha_unmasked_pairs(wl.cu_seqlens(), 0)
            print(json.dumps({"sweep_point": wl.name, "batch": len(wl.seqlens), "seq_len": wl.seqlens[0],
                              "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                              "kernel_avg_us": round(ms_kernel * 1e3, 2),
                              "frac": round(flops / (ms_kernel * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "graph_avg_us": round(ms_graph * 1e3, 2),
                              "frac_graph": round(flops / (ms_graph * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "steps": a.steps, "warmup": a.warmup,
                              "warmup_launches": warm_counts[wl.name]}), flush=True)
            torch.cuda.empty_cache()
        return

    name = a.workload or workloads.DEFAULT_BENCH_WORKLOAD
    wl = workloads.get(name)
    inp, ms_per_step, avg_ms, _ = timed(wl, a.steps, a.warmup, a.copy_calibration)

    pairs = tm.ts_mha_unmasked_pairs(wl.cu_seqlens(), wl.window)
    flops = 4 * wl.head_dim * wl.n_q_heads * pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    traffic = read_traffic(name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_launches": warm_counts[name],
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, fp32 sinks)",
        "config": {"workload": name, "seqlens": list(wl.seqlens) if len(wl.seqlens) <= 16 else None,
                   "total_tokens": wl.total_tokens, "n_q_heads": wl.n_q_heads,
                   "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "window": wl.window,
                   "sinks": wl.sinks, "softmax_scale": wl.softmax_scale},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "unmasked_pairs_per_head": pairs,
        "flops_per_step": flops,
        "kernel_avg_us": round(avg_ms * 1e3, 2),
        "algorithmic_GBps": round(algorithmic_bytes(wl) / (avg_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    line["per_launch"] = per_launch.get(name)
    # The vector ALU's roof: every visible score costs the softmax one v_mul_f32, one
    # v_exp_f32 and half a v_cvt_pk_bf16_f32; the microbenchmark gives the chip's rate of
    # exactly that mix at the kernel's occupancy.
    rates = ubench_rates(["softmax_score", "mfma_32x32x16_bf16"])
    scores = wl.n_q_heads * pairs
    line["roofline_valu"] = {"bound": "valu", "achieved": round(scores / (avg_ms * 1e-3) / 1e9, 1),
                             "peak": round(rates["softmax_score"]["scores_per_s"] / 1e9, 1),
                             "unit": "Gscore/s",
                             "frac": round(scores / (avg_ms * 1e-3) / rates["softmax_score"]["scores_per_s"], 4),
                             "per_score": "v_mul_f32 + v_exp_f32 + 1/2 v_cvt_pk_bf16_f32"}
    line["mfma_sustained_tflops"] = round(rates["mfma_32x32x16_bf16"]["tflops"], 1)
    line["device"] = device_info()
    if wl.window > 0:
        gbs = algorithmic_bytes(wl) / (avg_ms * 1e-3) / 1e9
        line["roofline_hbm"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "cache": "warm"}
        cold = cold_launch.get(name)
        if cold:
            cgbs = algorithmic_bytes(wl) / (cold["median_us"] * 1e-6) / 1e9
            line["roofline_hbm_cold"] = {"bound": "hbm", "achieved": round(cgbs, 1), "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": round(cgbs / PEAK_HBM_GBS, 4),
                                         "cache": f"cold: {a.flush_mib} MiB written before each launch",
                                         **cold}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, inp, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
