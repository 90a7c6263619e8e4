"""head_dim 128 in the two calls against a paged KV cache, vs the fp64 oracle's cache form.

ts_mha_decode_with_kvcache (the decode kernels at head_dim 128: 256-byte rows, two ring
stages per wave) and ts_mha_prefill_with_kvcache (the 128-row prefill kernel's paged
form) over every group size, page sizes 16..256, windows around tile edges, split
sequences and empty ones: the gate and the elementwise rounding bound against the
oracle; a whole sequence as the chunk equals ts_mha_prefill bit for bit; unused cache
slots (NaN) are never read.
"""
import numpy as np
import pytest
import torch

import sinks_ts_mha_amd as tm
from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import (cache_oracle_args, cache_rounding_bound, err_stats, f64, run_gpu, run_gpu_decode,
                   run_gpu_prefill_kv, say)
from test_gpu_prefill_kvcache import _paged_copy

pytestmark = pytest.mark.gpu

D = 128
SCALE = D ** -0.5
GATE_MAX, GATE_MEAN = 2e-2, 2e-3


def check(got, ref, what, bound):
    st = err_stats(got, ref)
    print(f"  {what}: max_abs={st['max_abs']:.3e} mean_abs={st['mean_abs']:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert st["max_abs"] <= GATE_MAX and st["mean_abs"] <= GATE_MEAN, f"{what}: gate {st}"
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"{what}: rounding bound exceeded by {excess.max():.3e}"


EDGES = [1, 15, 16, 17, 31, 32, 33, 0, 100, 1000]
DECODE_CASES = [
    # (k_lens, Hq, Hkv, page_size, window, sinks)
    (EDGES, 4, 4, 16, 0, True),            # G = 1
    (EDGES, 8, 4, 16, 0, True),            # G = 2
    (EDGES, 8, 2, 32, 0, False),           # G = 4
    (EDGES, 16, 2, 16, 0, True),           # G = 8
    (EDGES, 32, 2, 64, 0, True),           # G = 16
    (EDGES, 16, 2, 16, 1, True),
    (EDGES, 16, 2, 32, 127, True),
    (EDGES, 16, 2, 256, 129, False),
    ([300, 7, 4095, 4096, 4097], 16, 2, 16, 0, True),   # several chunks per sequence
    ([8192], 64, 8, 16, 0, True),                       # one long sequence split many ways
    ([9000, 130], 16, 1, 16, 1000, True),               # window spanning several chunks
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"c{n}" for n in range(len(DECODE_CASES))])
def test_decode_d128_parity(case, oracle_lib):
    k_lens, hq, hkv, page, w, sinks = case
    wl = workloads.decode(k_lens, n_q_heads=hq, n_kv_heads=hkv, window=w, page_size=page, sinks=sinks,
                          seed=31, head_dim=D, softmax_scale=SCALE)
    inp = workloads.make_cache_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0
    say(f"decode d128 k_lens={k_lens} Hq={hq} Hkv={hkv} page={page} W={w} sinks={sinks}")
    got = f64(run_gpu_decode(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"decode d128 k_lens={k_lens} G={hq // hkv} W={w}", cache_rounding_bound(inp, ref, oracle_lib))
    empty = [b for b, L in enumerate(k_lens) if L == 0]
    assert np.all(got[empty] == 0.0)


def test_decode_d128_batch_and_unused_slots(oracle_lib):
    """64 sequences of 2048 keys (the 64 x 8K decode shape, shorter) with spare pages: every
    element against the oracle, and NaN in every unused slot changes nothing."""
    wl = workloads.decode([2048] * 63 + [77], n_q_heads=64, n_kv_heads=8, page_size=16, seed=32,
                          head_dim=D, softmax_scale=SCALE, spare_pages=9)
    inp = workloads.make_cache_inputs(wl)
    say("decode d128 64 sequences, poisoned slots")
    clean = run_gpu_decode(inp).cpu()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(f64(clean), ref, "decode d128 64 x 2048", cache_rounding_bound(inp, ref, oracle_lib))
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


def test_decode_d128_noalloc_matches():
    """The decode call that allocates nothing gives the workspace call's result at head_dim 128."""
    wl = workloads.decode([20000, 300, 9000], n_q_heads=16, n_kv_heads=2, page_size=32, seed=33,
                          head_dim=D, softmax_scale=SCALE)
    inp = workloads.make_cache_inputs(wl)
    assert tm.ts_mha_decode_workspace_size(wl.n_seqs, 16, 2, D, 0, wl.max_seqlen_k) > 0
    say("decode d128 noalloc vs workspace")
    ref = run_gpu_decode(inp).cpu()
    dev = torch.device("cuda", 0)
    got = tm.ts_mha_decode_with_kvcache_noalloc(
        inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev), inp["sinks"].to(dev),
        inp["seqlens_k"].to(dev), inp["block_table"].to(dev), softmax_scale=SCALE,
        max_seqlen_k=wl.max_seqlen_k).cpu()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


RAGGED = [1, 63, 64, 65, 200, 517]
CHUNKS = ([1, 5, 64, 100, 33, 256], [300, 69, 1000, 100, 2000, 257])
PREFILL_CASES = [
    # (q_lens, k_lens, Hq, Hkv, page_size, window, sinks)
    (RAGGED, RAGGED, 16, 2, 16, 0, True),
    (*CHUNKS, 16, 2, 16, 0, True),          # G = 8
    (*CHUNKS, 8, 8, 16, 0, True),           # G = 1
    (*CHUNKS, 8, 4, 32, 0, False),          # G = 2
    (*CHUNKS, 8, 2, 64, 0, True),           # G = 4
    (*CHUNKS, 32, 2, 256, 0, True),         # G = 16
    (*CHUNKS, 16, 2, 16, 1, True),
    (*CHUNKS, 16, 2, 32, 128, True),
    (*CHUNKS, 16, 2, 16, 129, False),
    ([0, 3, 0, 7, 1], [10, 3, 0, 700, 1], 16, 2, 16, 0, True),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"c{n}" for n in range(len(PREFILL_CASES))])
def test_prefill_kvcache_d128_parity(case, oracle_lib):
    q_lens, k_lens, hq, hkv, page, w, sinks = case
    wl = workloads.CacheWorkload("t", tuple(q_lens), tuple(k_lens), hq, hkv, page, head_dim=D, window=w,
                                 sinks=sinks, softmax_scale=SCALE, seed=34)
    inp = workloads.make_cache_inputs(wl)
    if sinks:
        inp["sinks"] = inp["sinks"] * 2.0
    say(f"prefill-kv d128 q_lens={q_lens} k_lens={k_lens} Hq={hq} Hkv={hkv} page={page} W={w}")
    got = f64(run_gpu_prefill_kv(inp).cpu())
    torch.cuda.synchronize()
    ref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
    check(got, ref, f"prefill-kv d128 G={hq // hkv} page={page} W={w}", cache_rounding_bound(inp, ref, oracle_lib))


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_kvcache_d128_whole_chunk_equals_prefill(window):
    """Rows that are the whole sequence give ts_mha_prefill's head_dim 128 output bit for bit
    (unused page slots hold NaN)."""
    wl = workloads.custom([1, 63, 64, 65, 200, 517, 2048], 64, 8, window=window, head_dim=D,
                          softmax_scale=SCALE, seed=35)
    inp = workloads.make_inputs(wl)
    say(f"prefill-kv d128 whole chunk vs prefill, W={window}")
    a = run_gpu(inp).cpu()
    b = run_gpu_prefill_kv(_paged_copy(inp, 16, seed=5)).cpu()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_kvcache_d128_unused_slots_never_read():
    wl = workloads.CacheWorkload("t", (7, 300, 1), (900, 300, 33), 16, 2, 16, head_dim=D,
                                 softmax_scale=SCALE, seed=36, spare_pages=7)
    inp = workloads.make_cache_inputs(wl)
    say("prefill-kv d128 poisoned cache")
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
