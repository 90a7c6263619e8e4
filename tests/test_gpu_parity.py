"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Gate (every case): max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3 on
the bf16 outputs.  Small cases and the sampled rows of the long workloads also
pass a tighter elementwise bound derived from the kernel's roundings (bf16
probabilities, bf16 output, fp32 accumulation over the row's keys; see
_util.rounding_bound), which a wrong mask, sink or head mapping would break
where the gate cannot see it.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import assert_within_rounding, err_stats, f64, oracle_args, rounding_bound, run_gpu, say

pytestmark = pytest.mark.gpu

GATE_MAX, GATE_MEAN = 2e-2, 2e-3


def check(got, ref, what):
    st = err_stats(got, ref)
    print(f"  {what}: max_abs={st['max_abs']:.3e} mean_abs={st['mean_abs']:.3e} "
          f"ref_rms={st['ref_rms']:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert st["max_abs"] <= GATE_MAX, f"{what}: max abs err {st['max_abs']}"
    assert st["mean_abs"] <= GATE_MEAN, f"{what}: mean abs err {st['mean_abs']}"


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
    (RAGGED, 16, 2, 128, True),
    (RAGGED, 16, 2, 129, False),
    (RAGGED, 8, 1, 300, True),
    ([0, 1, 0, 5, 1, 0, 70], 16, 2, 0, True),
    ([1000], 64, 8, 0, True),
    ([777, 1], 32, 2, 64, True),
    (RAGGED, 1, 1, 0, True),       # a single head
    (RAGGED, 2, 1, 100, True),
    (RAGGED, 64, 64, 0, True),     # 64 KV heads (8 per XCD), G = 1
    (RAGGED, 128, 8, 129, True),   # 128 query heads, G = 16
]


@pytest.mark.parametrize("kernel", ["wide", "narrow"])
@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"c{n}" for n in range(len(SMALL_CASES))])
def test_small_parity(case, kernel, oracle_lib, monkeypatch):
    """Both head_dim 64 kernels (256- and 128-row work-groups), forced."""
    monkeypatch.setenv("TS_MHA_PREFILL_KERNEL", kernel)
    seqlens, hq, hkv, w, sinks = case
    wl = workloads.custom(seqlens, hq, hkv, window=w, sinks=sinks, seed=7)
    inp = workloads.make_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0  # wider spread of sink weights
    say(f"small parity ({kernel}) seqlens={seqlens} Hq={hq} Hkv={hkv} W={w} sinks={sinks}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.prefill(*oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"seqlens={seqlens} G={hq // hkv} W={w}")
    assert_within_rounding(got, inp, oracle_lib, what=f"seqlens={seqlens} W={w}")


FULL = ["tiny_1x128_gqa4", "gptoss_full_4x2048", "gptoss_window128_4x2048", "varlen16_window128",
        "gptoss_full_4x2048_kvgroup"]


@pytest.mark.parametrize("name", FULL)
def test_workload_parity_all_rows(name, oracle_lib):
    """Every output element of the workload, same launch as the benchmark's."""
    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    say(f"workload parity {name} T={wl.total_tokens}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.prefill(*oracle_args(inp), lib=oracle_lib)
    check(got, ref, name)


def test_long_prefill_sampled_rows(oracle_lib):
    """1 x 32768 full causal: rows sampled (the oracle would take far too long on all of them):
    positions 0..255, the last 64 positions and every 521st position, every query head."""
    wl = workloads.WORKLOADS["long_1x32768"]
    inp = workloads.make_inputs(wl)
    say("long prefill 1x32768 sampled rows")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    T = wl.total_tokens
    pos = np.unique(np.concatenate([np.arange(256), np.arange(T - 64, T), np.arange(0, T, 521)]))
    rows = np.repeat(pos, wl.n_q_heads)
    heads = np.tile(np.arange(wl.n_q_heads), pos.size)
    ref = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    check(got[rows, heads], ref, "long_1x32768 sampled")
    # The gate cannot see a dropped sink or a key too many on rows this long; the
    # elementwise bound (bf16 roundings, fp32 accumulation over up to 32768 keys) can.
    bound = rounding_bound(inp, ref, oracle_lib, rows=rows, heads=heads)
    excess = np.abs(got[rows, heads] - ref) - bound
    print(f"  long_1x32768 rounding bound: max excess {excess.max():.3e}, "
          f"max err/bound {(np.abs(got[rows, heads] - ref) / bound).max():.3f}", flush=True)
    assert excess.max() <= 0, f"rounding bound exceeded by {excess.max():.3e}"


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("n_seqs", [64, 256, 257])
def test_ragged_pack_sampled_rows(n_seqs, window, oracle_lib):
    """A large ragged pack at the GPT-OSS head shape: lengths uniform in [1, m] (seeded;
    m = 3000 for 64 sequences, 780 for more), so about half of the grid's position blocks
    are empty.  With 64 sequences the launch runs the compacted orders (by block level
    without a window, by sequence with one) over thousands of work-groups; with more, the
    direct order.  In every sequence the first 16 positions, the last 16 and every 509th,
    every query head, against the oracle's row routine, under the gate and the rounding
    bound."""
    rng = np.random.default_rng(37 + n_seqs)
    lens = rng.integers(1, (3001 if n_seqs <= 64 else 781), size=n_seqs).tolist()
    wl = workloads.custom(lens, 64, 8, window=window, seed=37)
    inp = workloads.make_inputs(wl)
    say(f"ragged pack n_seqs={n_seqs} W={window} T={wl.total_tokens}")
    out = run_gpu(inp).cpu()
    cu = wl.cu_seqlens().tolist()
    pos = []
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        rel = np.unique(np.concatenate([np.arange(min(16, L)), np.arange(max(0, L - 16), L), np.arange(0, L, 509)]))
        pos.append(cu[b] + rel)
    pos = np.concatenate(pos)
    rows = np.repeat(pos, wl.n_q_heads)
    heads = np.tile(np.arange(wl.n_q_heads), pos.size)
    got = f64(out[torch.from_numpy(rows), torch.from_numpy(heads)])
    ref = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    check(got, ref, f"ragged n_seqs={n_seqs} W={window}")
    excess = np.abs(got - ref) - rounding_bound(inp, ref, oracle_lib, rows=rows, heads=heads)
    assert excess.max() <= 0, f"rounding bound exceeded by {excess.max():.3e}"


# 1x1K, 2x1K and 1x2K run the 128-row kernel (their 256-row grids would leave CU slots empty)
SWEEP_CASES = ["sweep_b1_s1024", "sweep_b2_s1024", "sweep_b1_s2048", "sweep_b16_s1024",
               "sweep_b2_s4096", "sweep_b1_s8192", "sweep_b16_s8192"]


@pytest.mark.parametrize("name", SWEEP_CASES)
def test_chart_point_sampled_rows(name, oracle_lib):
    """Points of the chart family (sequence length x batch, full causal), at their real sizes
    and with the kernel the call picks for them: in every sequence the first 64 positions,
    the last 32 and every 257th, every query head."""
    wl = workloads.get(name)
    inp = workloads.make_inputs(wl)
    say(f"chart point {name} T={wl.total_tokens}")
    got = f64(run_gpu(inp).cpu())
    torch.cuda.synchronize()
    cu = wl.cu_seqlens().tolist()
    pos = []
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        rel = np.unique(np.concatenate([np.arange(64), np.arange(L - 32, L), np.arange(0, L, 257)]))
        pos.append(cu[b] + rel)
    pos = np.concatenate(pos)
    rows = np.repeat(pos, wl.n_q_heads)
    heads = np.tile(np.arange(wl.n_q_heads), pos.size)
    ref = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    check(got[rows, heads], ref, f"{name} sampled")
    excess = np.abs(got[rows, heads] - ref) - rounding_bound(inp, ref, oracle_lib, rows=rows, heads=heads)
    assert excess.max() <= 0, f"{name}: rounding bound exceeded by {excess.max():.3e}"


@pytest.mark.parametrize("head_dim,window", [(64, 0), (64, 128), (128, 0), (128, 128)])
def test_largest_accepted_sequence(head_dim, window, oracle_lib):
    """One sequence as long as the call accepts at 64 query / 8 KV heads: its query rows,
    plus one work-group's rows past the end, within 2^31 - 1 bytes (261887 tokens at
    head_dim 64, 130943 at 128; test_abi pins that one token more is refused).  Every
    32-bit buffer offset of the query, output and K/V rows reaches its largest value,
    and without a window the last rows walk the whole sequence.  The first 8 and last 8
    positions and 16 between, against the oracle's row routine under the gate and the
    rounding bound: every query head with the window, one per KV head without."""
    rows_past = 256 if head_dim == 64 else 128
    L = (2 ** 31 - 1) // (64 * 2 * head_dim) - rows_past
    wl = workloads.custom([L], 64, 8, window=window, head_dim=head_dim,
                          softmax_scale=head_dim ** -0.5, seed=43)
    inp = workloads.make_inputs(wl)
    say(f"largest sequence L={L} D={head_dim} W={window}")
    out = run_gpu(inp)
    pos = np.unique(np.concatenate([np.arange(8), np.arange(L - 8, L),
                                    np.linspace(8, L - 9, 16).astype(np.int64)]))
    if window:
        rows, heads = np.repeat(pos, 64), np.tile(np.arange(64), pos.size)
    else:
        rows = np.repeat(pos, 8)
        heads = np.tile(np.arange(8) * 8, pos.size) + np.repeat(pos % 8, 8)
    got = f64(out[torch.from_numpy(rows).to(out.device), torch.from_numpy(heads).to(out.device)])
    del out
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    check(got, ref, f"L={L} D={head_dim} W={window}")
    excess = np.abs(got - ref) - rounding_bound(inp, ref, oracle_lib, rows=rows, heads=heads)
    assert excess.max() <= 0, f"rounding bound exceeded by {excess.max():.3e}"
