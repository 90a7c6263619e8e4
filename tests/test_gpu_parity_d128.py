"""head_dim 128: the HIP path vs the fp64 oracle through the C ABI.

The same checks as at head_dim 64: the gate (max |err| <= 2e-2, mean <= 2e-3)
against the oracle, and on small cases the elementwise rounding bound against the
same oracle output; every element of two full-size workloads; the q = 0 closed
form at tight tolerance; the exact fallback on logits spread far beyond fp32's
range against reference 1; bitwise determinism, packing invariance and window
coverage; full overwrite of the output.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import assert_within_rounding, err_stats, f64, oracle_args, rounding_bound, run_gpu, say
from test_gpu_probes import q_zero_reference

pytestmark = pytest.mark.gpu

D = 128
SCALE = D ** -0.5
RAGGED = [1, 63, 64, 65, 200, 517]
SMALL_CASES = [
    # (seqlens, Hq, Hkv, window, sinks)
    (RAGGED, 8, 8, 0, True),       # G = 1
    (RAGGED, 8, 4, 0, True),       # G = 2
    (RAGGED, 8, 2, 0, False),      # G = 4
    (RAGGED, 16, 2, 0, True),      # G = 8
    (RAGGED, 32, 2, 0, True),      # G = 16
    (RAGGED, 16, 2, 1, True),
    (RAGGED, 16, 2, 127, True),
    (RAGGED, 16, 2, 128, False),
    (RAGGED, 32, 2, 129, True),
    (RAGGED, 8, 1, 300, True),
    ([0, 1, 0, 5, 1, 0, 70], 16, 2, 0, True),
    ([1000], 64, 8, 0, True),
]


def gate(got, ref, what):
    st = err_stats(got, ref)
    print(f"  {what}: max_abs={st['max_abs']:.3e} mean_abs={st['mean_abs']:.3e} "
          f"ref_rms={st['ref_rms']:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert st["max_abs"] <= 2e-2 and st["mean_abs"] <= 2e-3, what


@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"c{n}" for n in range(len(SMALL_CASES))])
def test_small_parity_d128(case, oracle_lib):
    seqlens, hq, hkv, w, sinks = case
    wl = workloads.custom(seqlens, hq, hkv, window=w, sinks=sinks, head_dim=D, softmax_scale=SCALE,
                          seed=17)
    inp = workloads.make_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0
    say(f"d128 small parity seqlens={seqlens} Hq={hq} Hkv={hkv} W={w} sinks={sinks}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    gate(got, oracle.prefill(*oracle_args(inp), lib=oracle_lib), f"seqlens={seqlens} W={w}")
    assert_within_rounding(got, inp, oracle_lib, what=f"d128 seqlens={seqlens} W={w}")


@pytest.mark.parametrize("name", list(workloads.D128_WORKLOADS))
def test_workload_parity_all_rows_d128(name, oracle_lib):
    wl = workloads.D128_WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    say(f"d128 workload parity {name} T={wl.total_tokens}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    gate(got, oracle.prefill(*oracle_args(inp), lib=oracle_lib), name)


@pytest.mark.parametrize("window", [0, 128])
def test_long_sequence_sampled_rows_d128(window, oracle_lib):
    """One 32768-token sequence at head_dim 128 (64 q / 8 KV heads, sinks; q and out 512 MiB
    each): up to 512 key tiles per work-group; positions 0-255, the last 64 and every 521st,
    every query head, against the oracle's row routine."""
    wl = workloads.custom([32768], 64, 8, window=window, head_dim=D, softmax_scale=SCALE, seed=0)
    inp = workloads.make_inputs(wl)
    say(f"d128 long sequence W={window} T={wl.total_tokens}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    L = wl.total_tokens
    pos = np.unique(np.concatenate([np.arange(256), np.arange(L - 64, L), np.arange(0, L, 521)]))
    rows = np.repeat(pos, wl.n_q_heads)
    heads = np.tile(np.arange(wl.n_q_heads), pos.size)
    ref = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    gate(got[rows, heads], ref.reshape(got[rows, heads].shape), f"d128 1x32768 W={window} sampled")
    # the elementwise bound, with fp32 accumulation over up to 32768 keys
    bound = rounding_bound(inp, ref, oracle_lib, rows=rows, heads=heads)
    excess = np.abs(got[rows, heads] - ref) - bound
    print(f"  d128 1x32768 W={window} rounding bound: max excess {excess.max():.3e}", flush=True)
    assert excess.max() <= 0, f"rounding bound exceeded by {excess.max():.3e}"


@pytest.mark.parametrize("window", [0, 1, 127, 128, 129])
def test_q_zero_closed_form_d128(window):
    """q = 0: every probability of a row is one number, so |err| <= 2^-7 |ref| (see the
    head_dim 64 probe); one key too many or too few moves a row far more."""
    wl = workloads.custom([2048, 300, 77], 64, 8, window=window, head_dim=D, softmax_scale=SCALE,
                          seed=18)
    inp = workloads.make_inputs(wl)
    inp["q"] = torch.zeros_like(inp["q"])
    inp["sinks"] = inp["sinks"] * 1.5
    say(f"d128 q=0 closed form W={window}")
    got = f64(run_gpu(inp).cpu())
    ref = q_zero_reference(inp)
    bound = 2.0 ** -7 * (1 + 2.0 ** -6) * np.abs(ref) + 1e-6
    assert np.all(np.abs(got - ref) <= bound), f"max excess {(np.abs(got - ref) - bound).max():.3e}"


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("sink", [None, 80.0, -80.0])
def test_fallback_and_sinks_d128(window, sink, oracle_lib):
    """Queries scaled by 40 (logits over hundreds of base-2 units) force the exact redo;
    sinks of +-80 push the row sums far from 1.  The elementwise bound and the gate
    against the oracle hold either way."""
    wl = workloads.custom([700, 333, 64, 5], 16, 2, window=window, head_dim=D, softmax_scale=SCALE,
                          seed=19)
    inp = workloads.make_inputs(wl)
    if sink is None:
        inp["q"] = (inp["q"].to(torch.float32) * 40.0).to(torch.bfloat16)
        inp["sinks"] = None
    else:
        inp["sinks"] = torch.full((16,), sink)
    say(f"d128 fallback/sinks W={window} sink={sink}")
    got = f64(run_gpu(inp).cpu())
    assert np.all(np.isfinite(got))
    assert_within_rounding(got, inp, oracle_lib, what=f"W={window} sink={sink}")
    if sink == 80.0:
        assert np.max(np.abs(got)) < 1e-6


def test_bitwise_invariants_d128():
    wl = workloads.custom([70, 1, 300, 129, 0, 64], 16, 2, window=100, head_dim=D,
                          softmax_scale=SCALE, seed=20)
    inp = workloads.make_inputs(wl)
    say("d128 packed vs alone, determinism, window coverage")
    packed = run_gpu(inp).cpu()
    again = run_gpu(inp).cpu()
    assert torch.equal(packed.view(torch.int16), again.view(torch.int16)), "run to run"
    cu = inp["cu_seqlens"].tolist()
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        one = dict(inp, q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e],
                   cu_seqlens=torch.tensor([0, e - s], dtype=torch.int32), max_seqlen=e - s)
        alone = run_gpu(one).cpu()
        assert torch.equal(alone.view(torch.int16), packed[s:e].view(torch.int16)), f"sequence {b}"
    full = run_gpu(inp, window=0).cpu()
    for w in (300, 2**31 - 1):
        wide = run_gpu(inp, window=w).cpu()
        assert torch.equal(full.view(torch.int16), wide.view(torch.int16)), f"W={w} >= L vs full"


def test_output_fully_overwritten_d128():
    wl = workloads.custom([257, 3, 1024], 16, 2, window=0, head_dim=D, softmax_scale=SCALE, seed=21)
    inp = workloads.make_inputs(wl)
    say("d128 output overwrite")
    T, hq = wl.total_tokens, wl.n_q_heads
    guard = 4096
    n = T * hq * D
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[guard:guard + n].view(T, hq, D)
    run_gpu(inp, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some output element was not written"
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all(), "guard band written"
