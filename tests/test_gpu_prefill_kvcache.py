"""Prefill of new rows against a paged KV cache: HIP path vs the fp64 oracle's cache form.

Gate (every case): max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3, plus the
elementwise rounding bound on the small cases, against the same oracle rows.  The cases cover chunks that are the whole
sequence, chunks at the end of a longer cache, single rows, every group size, page sizes
16..256, windows around tile edges and empty sequences; with the whole sequence as the chunk
the result must equal ts_mha_prefill on the same data bit for bit.
"""
import numpy as np
import pytest
import torch

import sinks_ts_mha_amd as tm
from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import (cache_oracle_args, cache_rounding_bound, err_stats, f64, run_gpu,
                   run_gpu_prefill_kv, say)

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


RAGGED = [1, 63, 64, 65, 200, 517]
CHUNKS = ([1, 5, 64, 100, 33, 256], [300, 69, 1000, 100, 2000, 257])
CASES = [
    # (q_lens, k_lens, Hq, Hkv, page_size, window, sinks)
    (RAGGED, RAGGED, 16, 2, 16, 0, True),
    (*CHUNKS, 16, 2, 16, 0, True),          # G = 8
    (*CHUNKS, 8, 8, 16, 0, True),           # G = 1
    (*CHUNKS, 8, 4, 32, 0, False),          # G = 2
    (*CHUNKS, 8, 2, 64, 0, True),           # G = 4
    (*CHUNKS, 32, 2, 256, 0, True),         # G = 16
    (*CHUNKS, 16, 2, 16, 1, True),
    (*CHUNKS, 16, 2, 16, 127, True),
    (*CHUNKS, 16, 2, 32, 128, True),
    (*CHUNKS, 16, 2, 16, 129, False),
    (*CHUNKS, 8, 1, 64, 300, True),
    ([0, 3, 0, 7, 1], [10, 3, 0, 700, 1], 16, 2, 16, 0, True),
    ([1, 1, 1], [5000, 17, 64], 16, 2, 16, 0, True),
    (*CHUNKS, 16, 2, 1024, 0, True),        # pages longer than a key tile or a query block
    (*CHUNKS, 64, 8, 2048, 100, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{n}" for n in range(len(CASES))])
def test_prefill_kvcache_small_parity(case, oracle_lib):
    q_lens, k_lens, hq, hkv, page, w, sinks = case
    wl = workloads.CacheWorkload("t", tuple(q_lens), tuple(k_lens), hq, hkv, page, window=w,
                                 sinks=sinks, seed=21)
    inp = workloads.make_cache_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0
    say(f"prefill-kv parity q_lens={q_lens} k_lens={k_lens} Hq={hq} Hkv={hkv} page={page} W={w}")
    got = f64(run_gpu_prefill_kv(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"q_lens={q_lens} G={hq // hkv} page={page} W={w}",
          bound=cache_rounding_bound(inp, ref, oracle_lib))


def _paged_copy(inp, page_size, seed):
    """The packed k/v of a prefill input dict, scattered into a shuffled page pool."""
    cu = inp["cu_seqlens"].tolist()
    n = len(cu) - 1
    need = [-(-(cu[b + 1] - cu[b]) // page_size) for b in range(n)]
    n_pages = sum(need) + 2
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    hkv, D = inp["k"].shape[1], inp["k"].shape[2]
    kc = torch.full((n_pages, page_size, hkv, D), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    table = torch.full((n, max(1, max(need))), -1, dtype=torch.int32)
    nxt = 0
    for b in range(n):
        for i in range(need[b]):
            pg = int(perm[nxt])
            nxt += 1
            table[b, i] = pg
            lo, hi = cu[b] + i * page_size, min(cu[b + 1], cu[b] + (i + 1) * page_size)
            kc[pg, :hi - lo] = inp["k"][lo:hi]
            vc[pg, :hi - lo] = inp["v"][lo:hi]
    lens = torch.tensor([cu[b + 1] - cu[b] for b in range(n)], dtype=torch.int32)
    return {"q": inp["q"], "k_cache": kc, "v_cache": vc, "sinks": inp["sinks"],
            "cu_seqlens_q": inp["cu_seqlens"], "seqlens_k": lens, "block_table": table,
            "max_seqlen_q": inp["max_seqlen"], "max_seqlen_k": inp["max_seqlen"],
            "page_size": page_size, "window": inp["window"], "softmax_scale": inp["softmax_scale"]}


@pytest.mark.parametrize("window", [0, 128])
def test_whole_sequence_chunk_equals_prefill(window):
    """Rows that are the whole sequence give ts_mha_prefill's output bit for bit (unused page
    slots hold NaN)."""
    wl = workloads.custom([1, 63, 64, 65, 200, 517, 2048], 64, 8, window=window, seed=22)
    inp = workloads.make_inputs(wl)
    say(f"prefill-kv whole chunk vs prefill, W={window}")
    a = run_gpu(inp).cpu()
    b = run_gpu_prefill_kv(_paged_copy(inp, 16, seed=3)).cpu()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_kvcache_unused_slots_never_read():
    wl = workloads.CacheWorkload("t", (7, 300, 1), (900, 300, 33), 16, 2, 16, seed=23, spare_pages=7)
    inp = workloads.make_cache_inputs(wl)
    say("prefill-kv poisoned cache")
    clean = run_gpu_prefill_kv(inp).cpu()
    used = torch.zeros(wl.n_pages, wl.page_size, dtype=torch.bool)
    for b, L in enumerate(wl.k_lens):
        for j in range(L):
            used[int(inp["block_table"][b, j // wl.page_size]), j % wl.page_size] = True
    kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
    kc[~used] = float("nan")
    vc[~used] = float("nan")
    dirty = run_gpu_prefill_kv(inp, k_cache=kc, v_cache=vc).cpu()
    torch.cuda.synchronize()
    assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16))


@pytest.mark.parametrize("name", list(workloads.PREFILL_KV_WORKLOADS))
def test_prefill_kvcache_workload_sampled_rows(name, oracle_lib):
    """The benchmark's chunked-prefill workloads, same launch as the benchmark: in every
    sequence the first 64 new rows, the last 32 and every 257th, every query head."""
    wl = workloads.PREFILL_KV_WORKLOADS[name]
    inp = workloads.make_cache_inputs(wl)
    say(f"prefill-kv workload {name}")
    got = f64(run_gpu_prefill_kv(inp).cpu())
    torch.cuda.synchronize()
    cu = inp["cu_seqlens_q"].tolist()
    pos = []
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        rel = np.unique(np.concatenate([np.arange(64), np.arange(L - 32, L), np.arange(0, L, 257)]))
        pos.append(cu[b] + rel)
    pos = np.concatenate(pos)
    rows = np.repeat(pos, wl.n_q_heads)
    heads = np.tile(np.arange(wl.n_q_heads), pos.size)
    ref = oracle.cache_attend(*cache_oracle_args(inp), rows=rows, heads=heads, lib=oracle_lib)
    check(got[rows, heads], ref, f"{name} sampled")


def test_prefill_kvcache_validate_mode(monkeypatch):
    wl = workloads.CacheWorkload("t", (8, 4), (40, 20), 8, 1, 16, seed=24)
    inp = workloads.make_cache_inputs(wl)
    say("prefill-kv TS_MHA_VALIDATE")
    monkeypatch.setenv("TS_MHA_VALIDATE", "1")
    run_gpu_prefill_kv(inp)
    short = dict(inp, seqlens_k=torch.tensor([40, 3], dtype=torch.int32))
    with pytest.raises(tm.TsMhaError) as e:
        run_gpu_prefill_kv(short)
    assert e.value.code == -9
    bad = dict(inp, block_table=inp["block_table"].clone())
    bad["block_table"][0, 2] = -5
    with pytest.raises(tm.TsMhaError) as e:
        run_gpu_prefill_kv(bad)
    assert e.value.code == -11
