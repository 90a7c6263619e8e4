"""Targeted GPU probes that the loose parity gate cannot see.

Closed forms at tight tolerance (window edges, sink units, head groups), edge
shapes, bitwise determinism and packing invariance, full overwrite of the
output, untouched guard bands, and the device checks of the C ABI.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import sinks_ts_mha_amd as tm
from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import assert_within_rounding, f64, oracle_args, run_gpu, say

pytestmark = pytest.mark.gpu


def q_zero_reference(inp):
    """q = 0: out_i = sum_{j in A_i} v_j / (|A_i| + e^sigma_h) (all logits are 0).

    When every probability of a row is the same number its bf16 rounding is one
    common relative error (at most u = 2^-8) and the output rounding another:
    |err| <= 2^-7 |ref| up to fp32 terms.  One key too many or too few moves a
    row by about 1 / sqrt(|A_i|) relative, far above that.
    """
    v = inp["v"].to(torch.float64).numpy()
    hq, hkv = inp["q"].shape[1], v.shape[1]
    G = hq // hkv
    w = inp["window"]
    cu = inp["cu_seqlens"].tolist()
    ref = np.zeros(inp["q"].shape)
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        cs = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v[s:e], axis=0)])
        i = np.arange(e - s)
        cnt = np.minimum(i + 1, w) if w > 0 else i + 1
        vsum = cs[i + 1] - cs[i + 1 - cnt]                          # [L, Hkv, D]
        for h in range(hq):
            extra = math.exp(float(inp["sinks"][h])) if inp["sinks"] is not None else 0.0
            ref[s:e, h] = vsum[:, h // G] / (cnt[:, None] + extra)
    return ref


Q_ZERO_CASES = [("gptoss_full_4x2048", 0), ("gptoss_window128_4x2048", 128),
                ("gptoss_window128_4x2048", 127), ("gptoss_window128_4x2048", 129),
                ("gptoss_window128_4x2048", 1)]


@pytest.mark.parametrize("name,window", Q_ZERO_CASES)
@pytest.mark.parametrize("sink_range", [(0.0, 3.0), (-3.0, 3.0)], ids=["sinks_nonneg", "sinks_mixed"])
def test_q_zero_closed_form(name, window, sink_range):
    """With q = 0 every logit of a row is 0, so every probability of the row is
    one number: exp(-sigma) against a sink reference, or 1.  All of them round
    alike, the rounded denominator carries the same relative error, and the
    output rounding adds u: |err| <= 2^-7 |ref|.  The negative-sink cases also
    get the general bound u (sum_j p_j |v_j| + 2 |out|), with sum_j p_j |v_j|
    given by the same closed form on |v|, should the reference differ between
    tiles."""
    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    inp["q"] = torch.zeros_like(inp["q"])
    inp["window"] = window
    inp["sinks"] = torch.linspace(sink_range[0], sink_range[1], wl.n_q_heads)
    say(f"q=0 closed form {name} W={window} sinks in {sink_range}")
    got = f64(run_gpu(inp).cpu())
    ref = q_zero_reference(inp)
    err = np.abs(got - ref)
    if sink_range[0] >= 0:
        bound = 2.0 ** -7 * (1 + 2.0 ** -6) * np.abs(ref) + 1e-5
    else:
        weighted_abs = q_zero_reference(dict(inp, v=inp["v"].abs()))
        bound = 2.0 ** -8 * (1 + 2.0 ** -6) * (weighted_abs + 2.0 * np.abs(ref)) + 1e-6
    if not np.all(err <= bound):
        excess = (err - bound).reshape(-1)
        cu = inp["cu_seqlens"].tolist()
        for flat in np.argsort(-excess)[:12]:
            t, h, d = np.unravel_index(flat, got.shape)
            b = int(np.searchsorted(cu, t, side="right")) - 1
            print(f"  token {t} (seq {b} pos {t - cu[b]}) head {h} d {d}: got {got[t, h, d]:.6e} "
                  f"ref {ref[t, h, d]:.6e} excess {excess[flat]:.3e}", flush=True)
        bad = (err > bound)
        print(f"  {bad.sum()} elements over; rows over per head: {bad.any(axis=2).sum(axis=0)}")
    assert np.all(err <= bound), f"max excess {(err - bound).max():.3e}"


@pytest.mark.parametrize("window", [1, 2, 3, 127, 128, 129])
def test_window_edges_tight(window, oracle_lib):
    wl = workloads.custom([300, 129, 128, 2], 16, 2, window=window, seed=3)
    inp = workloads.make_inputs(wl)
    say(f"window edge W={window}")
    got = f64(run_gpu(inp).cpu())
    assert_within_rounding(got, inp, oracle_lib)


@pytest.mark.parametrize("sink", [None, 0.0, 4.0, 80.0, -80.0])
def test_sink_values(sink, oracle_lib):
    wl = workloads.custom([500, 37], 16, 2, window=0, seed=4)
    inp = workloads.make_inputs(wl)
    inp["sinks"] = None if sink is None else torch.full((16,), sink)
    say(f"sink value {sink}")
    got = f64(run_gpu(inp).cpu())
    assert_within_rounding(got, inp, oracle_lib)
    if sink == 80.0:
        assert np.max(np.abs(got)) < 1e-6


@pytest.mark.parametrize("kernel", ["wide", "narrow"])
@pytest.mark.parametrize("seed", [6, 19])
@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("with_sinks", [True, False], ids=["sinks", "nosinks"])
def test_wide_logit_range(window, with_sinks, seed, kernel, oracle_lib, monkeypatch):
    """Queries scaled by 40 spread each row's logits over hundreds of log2 units,
    so measured against reference 1 many probabilities overflow fp32 (or their
    sums pass 2^64) in the fast pass.  Those work-groups must redo their rows
    with running maxima; every row still meets the rounding bound and the gate
    against the oracle on the same inputs.  With seed 19 some work-groups' row
    sums come out NaN (an infinite probability times a zero of the row-sum
    selector): the range test must catch NaN too."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([700, 333, 64, 5], 16, 2, window=window, seed=seed)
    inp = workloads.make_inputs(wl)
    inp["q"] = (inp["q"].to(torch.float32) * 40.0).to(torch.bfloat16)
    if not with_sinks:
        inp["sinks"] = None
    say(f"wide logit range window={window} sinks={with_sinks} seed={seed}")
    got = f64(run_gpu(inp).cpu())
    assert np.all(np.isfinite(got))
    assert_within_rounding(got, inp, oracle_lib, what=f"W={window} sinks={with_sinks} seed={seed}")


@pytest.mark.parametrize("head_dim,kernel", [(64, "wide"), (64, "narrow"), (128, "narrow")])
@pytest.mark.parametrize("spread", [2.0, 4.0, 8.0, 16.0])
def test_logit_spread_gate(spread, head_dim, kernel, oracle_lib, monkeypatch):
    """Queries scaled by 2 .. 16 make attention ever more peaked (logit standard deviation
    2 .. 16 at scale 1/sqrt(head_dim)), the range where trained attention lives.  The
    kernels take q.k exactly (bf16 products, fp32 sums) and apply the scale in fp32, so no
    rounding of the logits grows with their spread: the rounding bound and the gate hold
    against the oracle on the original inputs at every spread."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([700, 333, 64, 5], 16, 2, window=0, head_dim=head_dim,
                          softmax_scale=head_dim ** -0.5, seed=23)
    inp = workloads.make_inputs(wl)
    inp["q"] = (inp["q"].to(torch.float32) * spread).to(torch.bfloat16)
    say(f"logit spread x{spread} D={head_dim} {kernel}")
    got = f64(run_gpu(inp).cpu())
    assert np.all(np.isfinite(got))
    assert_within_rounding(got, inp, oracle_lib, what=f"spread x{spread} D={head_dim} {kernel}")


def test_edge_shapes(oracle_lib):
    for seqlens in ([0], [1], [0, 0], [1, 0, 2, 0], [5]):
        wl = workloads.custom(seqlens, 8, 1, window=0, seed=5)
        inp = workloads.make_inputs(wl)
        say(f"edge shape {seqlens}")
        got = run_gpu(inp)
        torch.cuda.synchronize()
        if wl.total_tokens:
            assert_within_rounding(f64(got.cpu()), inp, oracle_lib)


def test_no_sequences_is_noop():
    """n_seqs = 0 (and max_seqlen = 0) is accepted and launches nothing."""
    q = torch.zeros(16, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(16, 1, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("n_seqs = 0")
    for max_len in (0, 16):
        rc = tm.lib().ts_mha_prefill(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, cu.data_ptr(),
                                     8, 1, 64, 0, 0.125, out.data_ptr(), 0, max_len, None)
        assert rc == 0
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


@pytest.mark.parametrize("kernel", ["auto", "wide", "narrow"])
@pytest.mark.parametrize("window", [0, 100])
def test_packed_equals_alone_bitwise(window, kernel, monkeypatch):
    """A sequence's rows do not depend on the sequences packed with it.  The ragged
    pack has most of its grid's position blocks empty, so the kernels run it in their
    compacted orders (by sequence with a window, by block index without); a sequence
    alone fills its grid and takes the direct order."""
    if kernel != "auto":
        monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([70, 1, 300, 129, 0, 64, 1000], 16, 2, window=window, seed=6)
    inp = workloads.make_inputs(wl)
    say(f"packed vs alone W={window} {kernel}")
    packed = run_gpu(inp).cpu()
    cu = inp["cu_seqlens"].tolist()
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        one = dict(inp, q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e],
                   cu_seqlens=torch.tensor([0, e - s], dtype=torch.int32), max_seqlen=e - s)
        alone = run_gpu(one).cpu()
        assert torch.equal(alone.view(torch.int16), packed[s:e].view(torch.int16)), f"sequence {b}"


@pytest.mark.parametrize("shape,check", [
    (([8192] * 3, 0, 64), None),               # groups of 2 sequences: {0, 1}, {2}
    (([4096] * 5 + [4000], 128, 64), None),    # groups of 4: {0..3}, {4, 5}
    (([1024] * 70, 0, 64), [0, 15, 16, 31, 47, 63, 64, 69]),  # groups of 16, the last of 6
    (([4096] * 5, 0, 128), None),              # head_dim 128, groups of 2: {0, 1}, {2, 3}, {4}
    (([2048] * 9, 100, 128), [0, 3, 4, 7, 8]),  # head_dim 128, groups of 4, the last of 1
], ids=["3x8192", "6x4096_w128", "70x1024", "d128_5x4096", "d128_9x2048_w100"])
def test_sequence_groups_packed_equals_alone(shape, check):
    """Uniform batches run in the direct order, which takes the sequences in groups whose
    K and V fit one XCD's L2 (4 MiB: at 8 KV heads and head_dim 64, 2 sequences of 8192
    tokens, 4 of 4096, 16 of 1024; half as many at head_dim 128), the last group smaller.
    Every row of the batch, written over NaN, equals its sequence run alone bit for bit (a
    block left out or run twice or at the wrong sequence would differ)."""
    (seqlens, w, d) = shape
    wl = workloads.custom(seqlens, 64, 8, window=w, head_dim=d, softmax_scale=d ** -0.5, seed=21)
    inp = workloads.make_inputs(wl)
    say(f"sequence groups {len(seqlens)} x {max(seqlens)} W={w} D={d}")
    dev = torch.device("cuda", 0)
    out = torch.full(inp["q"].shape, float("nan"), dtype=torch.bfloat16, device=dev)
    packed = run_gpu(inp, out=out).cpu()
    cu = inp["cu_seqlens"].tolist()
    for b in (range(len(seqlens)) if check is None else check):
        s, e = cu[b], cu[b + 1]
        one = dict(inp, q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e],
                   cu_seqlens=torch.tensor([0, e - s], dtype=torch.int32), max_seqlen=e - s)
        alone = run_gpu(one).cpu()
        assert torch.equal(alone.view(torch.int16), packed[s:e].view(torch.int16)), f"sequence {b}"
    assert not torch.isnan(packed).any()


@pytest.mark.parametrize("qscale", [1.0, 40.0], ids=["fast", "redo"])
@pytest.mark.parametrize("shape", [([70, 1, 300, 129, 0, 64], 16, 2, 100), ([1000, 333], 64, 8, 0),
                                   ([2048] * 2, 64, 8, 128), ([517, 65, 1], 32, 2, 0), ([300], 8, 8, 0)],
                         ids=["ragged_w100", "g8", "g8_w128", "g16", "g1"])
def test_wide_and_narrow_kernels_agree_bitwise(shape, qscale, monkeypatch):
    """At head_dim 64 the launch picks the 256- or the 128-row work-groups by grid
    size; for each row both walk its visible keys with the same instructions in the
    same order (the extra keys either kind covers are masked or skipped and add exact
    zeros), so their outputs are identical bit for bit.  Queries scaled by 40 make some
    work-groups redo their rows exactly; the 256-row kernel decides that per half of
    its rows, which are the rows of one 128-row work-group, so the redo does not break
    the equality either."""
    seqlens, hq, hkv, w = shape
    wl = workloads.custom(seqlens, hq, hkv, window=w, seed=12)
    inp = workloads.make_inputs(wl)
    inp["q"] = (inp["q"].to(torch.float32) * qscale).to(torch.bfloat16)
    say(f"wide vs narrow {shape} q x{qscale}")
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", "wide")
    a = run_gpu(inp).cpu()
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", "narrow")
    b = run_gpu(inp).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("window", [0, 64])
@pytest.mark.parametrize("n_seqs", [70, 256, 257])
def test_many_sequences(n_seqs, window, oracle_lib):
    """Many short sequences (lengths 1 .. 300), more than the compacted orders serve (64):
    the direct order with its empty blocks, against the oracle."""
    rng = np.random.default_rng(36 + n_seqs)
    wl = workloads.custom(rng.integers(1, 301, size=n_seqs).tolist(), 16, 2, window=window, seed=36)
    inp = workloads.make_inputs(wl)
    say(f"{n_seqs} sequences W={window}")
    assert_within_rounding(f64(run_gpu(inp).cpu()), inp, oracle_lib, what=f"{n_seqs} sequences W={window}")


@pytest.mark.parametrize("kernel", ["wide", "narrow"])
@pytest.mark.parametrize("window", [0, 128])
def test_max_seqlen_only_sizes_the_grid(window, kernel, monkeypatch):
    """max_seqlen bounds the sequence lengths and sizes the grid, nothing more: a bound
    4x too large (three quarters of the grid empty, so the compacted orders run) or
    exactly 1 past the longest sequence gives the exact bound's output bit for bit."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([512, 512, 300, 512], 64, 8, window=window, seed=38)
    inp = workloads.make_inputs(wl)
    say(f"max_seqlen padding W={window} {kernel}")
    ref = run_gpu(inp).cpu()
    for m in (513, 2048):
        got = run_gpu(dict(inp, max_seqlen=m)).cpu()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"max_seqlen={m}"


def test_deterministic_bitwise():
    wl = workloads.WORKLOADS["gptoss_full_4x2048"]
    inp = workloads.make_inputs(wl)
    say("determinism")
    a = run_gpu(inp).cpu()
    b = run_gpu(inp).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_window_covering_equals_full_bitwise():
    wl = workloads.custom([1000, 333], 16, 2, window=0, seed=8)
    inp = workloads.make_inputs(wl)
    say("window >= length vs full")
    full = run_gpu(inp).cpu()
    # 2^31 - 1 also takes the mask's window arithmetic through its wrap-around
    for w in (1000, 5000, 2**31 - 1):
        got = run_gpu(inp, window=w).cpu()
        assert torch.equal(got.view(torch.int16), full.view(torch.int16)), f"W={w}"


@pytest.mark.parametrize("kernel", ["wide", "narrow"])
@pytest.mark.parametrize("window", [0, 100])
def test_output_fully_overwritten_and_guards_intact(window, kernel, monkeypatch):
    """Every output element is written and nothing outside the output is.  The ragged
    pack leaves most of its grid's blocks empty, so this also checks that the compacted
    orders give every block of every sequence to exactly one work-group."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([257, 3, 1024, 0, 65], 16, 2, window=window, seed=9)
    inp = workloads.make_inputs(wl)
    n = inp["q"].numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[guard:guard + n].view(inp["q"].shape)
    say(f"NaN-poisoned output with guard bands W={window} {kernel}")
    run_gpu(inp, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some output element was not written"
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all(), "guard band written"


def test_runs_on_a_side_stream(oracle_lib):
    wl = workloads.custom([300, 40], 16, 2, window=0, seed=11)
    inp = workloads.make_inputs(wl)
    say("side stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run_gpu(inp, stream=s)
    s.synchronize()
    assert_within_rounding(f64(got.cpu()), inp, oracle_lib)


@pytest.mark.parametrize("head_dim,kernel,window", [(64, "wide", 0), (64, "narrow", 0),
                                                     (64, "wide", 128), (128, "narrow", 100)])
def test_graph_replay_matches_eager(head_dim, kernel, window, monkeypatch):
    """A prefill call captured in a HIP graph gives the eager result bit for bit on every
    replay, with other eager work and synchronisations between replays (the library records
    no memset node and keeps no state between calls)."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    wl = workloads.custom([700, 1, 2048, 65], 64, 8, window=window, head_dim=head_dim,
                          softmax_scale=head_dim ** -0.5, seed=14)
    inp = workloads.make_inputs(wl)
    say(f"graph replay D={head_dim} {kernel} W={window}")
    dev = torch.device("cuda", 0)
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    sinks, cu = inp["sinks"].to(dev), inp["cu_seqlens"].to(dev)
    kw = dict(window=window, softmax_scale=wl.softmax_scale, max_seqlen=wl.max_seqlen)
    eager = tm.ts_mha_prefill(q, k, v, sinks, cu, **kw).clone()
    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            tm.ts_mha_prefill(q, k, v, sinks, cu, out=out, **kw)
    for rep in range(3):
        out.fill_(float("nan"))
        other = tm.ts_mha_prefill(q, k, v, sinks, cu, **kw)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16)), f"eager {rep}"
    del graph


def test_arch_check_hook(monkeypatch):
    q = torch.zeros(4, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(4, 1, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("TS_MHA_TEST_ARCH", "gfx942")
    say("arch hook")
    with pytest.raises(tm.TsMhaError) as ei:
        tm.ts_mha_prefill(q, k, k.clone(), None, cu, max_seqlen=4)
    assert ei.value.code == -7


def test_debug_seqlens_validation(monkeypatch):
    q = torch.zeros(8, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(8, 1, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 3, 8], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("TS_MHA_VALIDATE", "1")
    say("debug cu_seqlens validation")
    with pytest.raises(tm.TsMhaError) as ei:
        tm.ts_mha_prefill(q, k, k.clone(), None, cu, max_seqlen=4)   # length 5 > 4
    assert ei.value.code == -9
    tm.ts_mha_prefill(q, k, k.clone(), None, cu, max_seqlen=5)
    torch.cuda.synchronize()


def test_binding_rejects_overlapping_out():
    """The binding refuses an output that shares bytes with any input (the kernels read the
    inputs while they write the output), and accepts an adjacent, non-overlapping one."""
    wl = workloads.custom([64, 64], 16, 2, seed=22)
    inp = workloads.make_inputs(wl, device="cuda")
    q, k, v, s, cu = inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"]
    say("binding overlap checks")
    n, bf = q.numel(), torch.bfloat16
    buf = torch.empty(2 * n, dtype=bf, device="cuda")  # q, then room for an output
    qq = buf[:n].view(q.shape)
    qq.copy_(q)
    with pytest.raises(ValueError, match="overlap"):
        tm.ts_mha_prefill(qq, k, v, s, cu, out=qq, max_seqlen=64)
    with pytest.raises(ValueError, match="overlap"):
        tm.ts_mha_prefill(qq, k, v, s, cu, out=buf[n // 2: n // 2 + n].view(q.shape), max_seqlen=64)
    kbuf = torch.empty(n, dtype=bf, device="cuda")  # k inside the output's bytes
    kk = kbuf[: k.numel()].view(k.shape)
    kk.copy_(k)
    with pytest.raises(ValueError, match="overlap"):
        tm.ts_mha_prefill(q, kk, v, s, cu, out=kbuf.view(q.shape), max_seqlen=64)
    sbuf = torch.empty(n, dtype=bf, device="cuda")  # the sinks inside the output's bytes
    ss = sbuf[: 2 * s.numel()].view(torch.float32)
    ss.copy_(s)
    with pytest.raises(ValueError, match="overlap"):
        tm.ts_mha_prefill(q, k, v, ss, cu, out=sbuf.view(q.shape), max_seqlen=64)
    dwl = workloads.decode([40, 7], n_q_heads=16, n_kv_heads=2, page_size=16, seed=23)
    dinp = workloads.make_cache_inputs(dwl)
    dq = dinp["q"].cuda()
    with pytest.raises(ValueError, match="overlap"):
        tm.ts_mha_decode_with_kvcache(dq, dinp["k_cache"].cuda(), dinp["v_cache"].cuda(), dinp["sinks"].cuda(),
                                      dinp["seqlens_k"].cuda(), dinp["block_table"].cuda(), out=dq,
                                      max_seqlen_k=dwl.max_seqlen_k)
    out = buf[n:].view(q.shape)  # adjacent to q, not overlapping
    tm.ts_mha_prefill(qq, k, v, s, cu, out=out, max_seqlen=64)
    ref = tm.ts_mha_prefill(q, k, v, s, cu, max_seqlen=64)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
