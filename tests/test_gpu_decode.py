"""Decode against a paged KV cache: HIP path vs the fp64 oracle's cache form, through the C ABI.

Gate (every case): max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3 on the bf16
outputs, plus the elementwise rounding bound of the kernel's roundings on the small cases.
Shapes cover every group size, page sizes 16..256, windows at and around tile edges, cached
lengths at tile and page edges, empty sequences, and sequences long enough to be split into
key chunks that a second kernel merges.
"""
import os

import numpy as np
import pytest
import torch

import sinks_ts_mha_amd as tm
from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import cache_oracle_args, cache_rounding_bound, err_stats, f64, run_gpu_decode, say

pytestmark = pytest.mark.gpu

GATE_MAX, GATE_MEAN = 2e-2, 2e-3


def check(got, ref, what, bound=None):
    st = err_stats(got, ref)
    print(f"  {what}: max_abs={st['max_abs']:.3e} mean_abs={st['mean_abs']:.3e} "
          f"ref_rms={st['ref_rms']:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert st["max_abs"] <= GATE_MAX, f"{what}: max abs err {st['max_abs']}"
    assert st["mean_abs"] <= GATE_MEAN, f"{what}: mean abs err {st['mean_abs']}"
    if bound is not None:
        excess = np.abs(got - ref) - bound
        assert excess.max() <= 0, f"{what}: rounding bound exceeded by {excess.max():.3e}"


EDGES = [1, 15, 16, 17, 31, 32, 33, 0, 100, 1000]
CASES = [
    # (k_lens, Hq, Hkv, page_size, window, sinks)
    (EDGES, 4, 4, 16, 0, True),            # G = 1
    (EDGES, 8, 4, 16, 0, True),            # G = 2
    (EDGES, 8, 2, 32, 0, False),           # G = 4
    (EDGES, 16, 2, 16, 0, True),           # G = 8
    (EDGES, 32, 2, 64, 0, True),           # G = 16
    (EDGES, 16, 2, 16, 1, True),
    (EDGES, 16, 2, 16, 5, True),
    (EDGES, 16, 2, 32, 127, True),
    (EDGES, 16, 2, 16, 128, True),
    (EDGES, 16, 2, 256, 129, False),
    ([300, 7, 4095, 4096, 4097], 16, 2, 16, 0, True),   # several chunks per sequence
    ([8192], 64, 8, 16, 0, True),                       # one long sequence: 64 chunks
    ([5000, 2, 3001], 4, 4, 64, 0, True),
    ([9000, 130], 16, 1, 16, 1000, True),               # window spanning several chunks
    (EDGES, 1, 1, 16, 0, True),            # a single head
    (EDGES, 64, 64, 16, 0, True),          # 64 KV heads, G = 1: two per work-group
    (EDGES, 128, 8, 32, 100, True),        # 128 query heads, G = 16
    ([5000, 17, 2048, 0, 4097], 16, 2, 2048, 0, True),  # pages longer than a key chunk
    ([5000, 17, 2048, 0, 4097], 32, 8, 1024, 300, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{n}" for n in range(len(CASES))])
def test_decode_small_parity(case, oracle_lib):
    k_lens, hq, hkv, page, w, sinks = case
    wl = workloads.decode(k_lens, n_q_heads=hq, n_kv_heads=hkv, window=w, page_size=page,
                          sinks=sinks, seed=11)
    inp = workloads.make_cache_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0
    say(f"decode parity k_lens={k_lens} Hq={hq} Hkv={hkv} page={page} W={w} sinks={sinks}")
    got = f64(run_gpu_decode(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"k_lens={k_lens} G={hq // hkv} page={page} W={w}",
          bound=cache_rounding_bound(inp, ref, oracle_lib))
    empty = [b for b, L in enumerate(k_lens) if L == 0]
    assert np.all(got[empty] == 0.0), "a sequence without keys must give zero rows"


@pytest.mark.parametrize("name", list(workloads.DECODE_WORKLOADS))
def test_decode_workload_parity(name, oracle_lib):
    """Every output element of the benchmark's decode workloads, same launch as the benchmark."""
    wl = workloads.DECODE_WORKLOADS[name]
    inp = workloads.make_cache_inputs(wl)
    say(f"decode workload parity {name}")
    got = f64(run_gpu_decode(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, name)


def test_decode_unused_slots_never_read():
    """NaN in every slot no sequence uses (spare pages, slots past each sequence's end) and -1
    in unused block-table entries change nothing, bit for bit."""
    wl = workloads.decode([37, 16, 1, 300, 0, 4100], n_q_heads=16, n_kv_heads=2, page_size=16,
                          seed=12, spare_pages=9)
    inp = workloads.make_cache_inputs(wl)
    say("decode poisoned cache")
    clean = run_gpu_decode(inp).cpu()
    used = torch.zeros(wl.n_pages, wl.page_size, dtype=torch.bool)
    for b, L in enumerate(wl.k_lens):
        for j in range(L):
            used[int(inp["block_table"][b, j // wl.page_size]), j % wl.page_size] = True
    kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
    kc[~used] = float("nan")
    vc[~used] = float("nan")
    dirty = run_gpu_decode(inp, k_cache=kc, v_cache=vc).cpu()
    torch.cuda.synchronize()
    assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16))


def test_decode_run_to_run_and_side_stream():
    wl = workloads.decode([8192, 33, 2048], n_q_heads=64, n_kv_heads=8, page_size=16, seed=13)
    inp = workloads.make_cache_inputs(wl)
    say("decode determinism, explicit workspace, side stream")
    a = run_gpu_decode(inp).cpu()
    need = tm.ts_mha_decode_workspace_size(wl.n_seqs, 64, 8, 64, 0, wl.max_seqlen_k)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage contents
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        b = run_gpu_decode(inp, workspace=ws, stream=side)
    side.synchronize()
    assert torch.equal(a.view(torch.int16), b.cpu().view(torch.int16))


def test_decode_out_fully_overwritten():
    wl = workloads.decode([0, 1, 77, 0], n_q_heads=16, n_kv_heads=2, page_size=16, seed=14)
    inp = workloads.make_cache_inputs(wl)
    say("decode NaN-poisoned output")
    dev = torch.device("cuda", 0)
    guard = torch.full((inp["q"].numel() + 2 * 4096,), float("nan"), dtype=torch.bfloat16, device=dev)
    out = guard[4096:4096 + inp["q"].numel()].view(inp["q"].shape)
    run_gpu_decode(inp, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.isnan(guard[:4096]).all() and torch.isnan(guard[-4096:]).all()
    assert torch.all(out[0] == 0) and torch.all(out[3] == 0)


def test_decode_validate_mode(monkeypatch):
    wl = workloads.decode([40, 20], n_q_heads=8, n_kv_heads=1, page_size=16, seed=15)
    inp = workloads.make_cache_inputs(wl)
    say("decode TS_MHA_VALIDATE")
    monkeypatch.setenv("TS_MHA_VALIDATE", "1")
    run_gpu_decode(inp)  # a valid call passes
    bad = dict(inp, block_table=inp["block_table"].clone())
    bad["block_table"][1, 0] = wl.n_pages
    with pytest.raises(tm.TsMhaError) as e:
        run_gpu_decode(bad)
    assert e.value.code == -11
    long = dict(inp, seqlens_k=torch.tensor([40, 33], dtype=torch.int32), max_seqlen_k=32)
    with pytest.raises(tm.TsMhaError) as e:
        run_gpu_decode(long)
    assert e.value.code == -9


def test_decode_graph_replay_matches_eager():
    """A decode call captured in a HIP graph gives the eager result on every replay, with
    other eager work between replays (the library records no memset node)."""
    wl = workloads.decode([8192, 5, 700], n_q_heads=64, n_kv_heads=8, page_size=16, seed=16)
    inp = workloads.make_cache_inputs(wl)
    say("decode graph replay")
    dev = torch.device("cuda", 0)
    q, kc, vc = inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    sinks, lens, table = inp["sinks"].to(dev), inp["seqlens_k"].to(dev), inp["block_table"].to(dev)
    need = tm.ts_mha_decode_workspace_size(wl.n_seqs, 64, 8, 64, 0, wl.max_seqlen_k)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    eager = tm.ts_mha_decode_with_kvcache(q, kc, vc, sinks, lens, table, max_seqlen_k=wl.max_seqlen_k,
                                          softmax_scale=0.125, workspace=ws).clone()
    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            tm.ts_mha_decode_with_kvcache(q, kc, vc, sinks, lens, table, max_seqlen_k=wl.max_seqlen_k,
                                          softmax_scale=0.125, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


HEAD_GROUP_CASES = [
    # (k_lens rng spec (n_seqs, max len, share empty), Hq, Hkv, head_dim, window): the KV heads
    # per work-group and whether sequences are split follow from the shapes
    ((256, 300, 0.1), 16, 4, 64, 0),      # 4 heads per work-group, 256 work-groups, no split
    ((128, 300, 0.1), 16, 4, 64, 33),     # 2 heads per work-group (4 would leave CUs idle)
    ((86, 200, 0.1), 12, 6, 64, 0),       # 6 KV heads: 2 per work-group
    ((256, 150, 0.2), 32, 2, 128, 0),     # head_dim 128, G = 16: 2 heads, 512 output chunks
    ((256, 150, 0.2), 16, 2, 128, 100),
    ((4, 9000, 0.25), 32, 4, 64, 2500),   # long windowed spans: 4 heads and split chunks
    ((3, 6000, 0.0), 8, 8, 128, 0),       # head_dim 128, G = 1: 2 heads and split chunks
    ((3, 5000, 0.0), 8, 4, 64, 0),        # 4 heads of G = 2, split chunks
    ((3, 5000, 0.0), 16, 4, 64, 3000),    # 4 heads of G = 4, a window over several chunks
    ((4, 9000, 0.0), 64, 4, 64, 0),       # 4 heads of G = 16
]


@pytest.mark.parametrize("case", HEAD_GROUP_CASES, ids=[f"hg{n}" for n in range(len(HEAD_GROUP_CASES))])
def test_decode_head_groups(case, oracle_lib):
    """Work-groups that serve several adjacent KV heads (their waves split between the heads),
    with and without split sequences: against the oracle under the gate and the rounding
    bound, empty sequences give zero rows, and nothing outside the output is written."""
    (n, max_len, p_empty), hq, hkv, d, w = case
    rng = np.random.default_rng(71 + n + d + w)
    k_lens = rng.integers(1, max_len + 1, size=n)
    k_lens[rng.random(n) < p_empty] = 0
    k_lens = k_lens.tolist()
    wl = workloads.decode(k_lens, n_q_heads=hq, n_kv_heads=hkv, window=w, page_size=16, seed=72,
                          head_dim=d, softmax_scale=d ** -0.5)
    inp = workloads.make_cache_inputs(wl)
    inp["sinks"] = inp["sinks"] * 2.0
    say(f"decode head groups n_seqs={n} Hq={hq} Hkv={hkv} D={d} W={w}")
    dev = torch.device("cuda", 0)
    guard = torch.full((inp["q"].numel() + 2 * 4096,), float("nan"), dtype=torch.bfloat16, device=dev)
    out = guard[4096:4096 + inp["q"].numel()].view(inp["q"].shape)
    run_gpu_decode(inp, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(guard[:4096]).all() and torch.isnan(guard[-4096:]).all()
    got = f64(out.cpu())
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"n_seqs={n} G={hq // hkv} D={d} W={w}", bound=cache_rounding_bound(inp, ref, oracle_lib))
    empty = [b for b, L in enumerate(k_lens) if L == 0]
    assert np.all(got[empty] == 0.0), "a sequence without keys must give zero rows"


def test_decode_million_keys(oracle_lib):
    """Sequences of 2^20 and 2^19 + 5 cached keys beside a 3-key one (64 q / 8 KV heads,
    page 16: 98 306 pages spread at random over the pool): page ids and byte offsets far
    into a 3 GiB cache, 128 key chunks per sequence merged, against the oracle's cache
    form under the gate and the rounding bound."""
    wl = workloads.decode([1 << 20, 3, (1 << 19) + 5], n_q_heads=64, n_kv_heads=8, page_size=16, seed=73)
    inp = workloads.make_cache_inputs(wl)
    say("decode 2^20 cached keys")
    got = f64(run_gpu_decode(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, "2^20 keys", bound=cache_rounding_bound(inp, ref, oracle_lib))
