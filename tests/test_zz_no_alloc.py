"""The decode entry point that allocates nothing, against the one with a caller's workspace.

ts_mha_decode_with_kvcache_noalloc keeps the partial results of split sequences in the
library's own per-GPU scratch array instead of a workspace.  Called through the C ABI,
it must give exactly the output of ts_mha_decode_with_kvcache (same kernels, same
split), on two calls in a row where the second has a smaller input (the scratch keeps
the first call's contents), and the oracle's output within the rounding bound.  A
split needing more than the scratch holds is refused on the host.
"""
import numpy as np
import pytest
import torch

import sinks_ts_mha_amd as tm
from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import cache_oracle_args, cache_rounding_bound, f64, run_gpu_decode, say

# (k_lens, Hq, Hkv, page_size, window): both split every sequence into chunks, so the
# scratch is in use; the second is smaller in every dimension.
CALLS = [([20000, 9000, 15000, 300], 64, 8, 16, 0),
         ([5000, 70], 16, 2, 32, 0)]


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode(oracle_lib):
    dev = torch.device("cuda", 0)
    for n, (k_lens, hq, hkv, page, w) in enumerate(CALLS):
        wl = workloads.decode(k_lens, n_q_heads=hq, n_kv_heads=hkv, window=w, page_size=page,
                              seed=40 + n)
        inp = workloads.make_cache_inputs(wl)
        need = tm.ts_mha_decode_workspace_size(wl.n_seqs, hq, hkv, 64, w, wl.max_seqlen_k)
        assert 0 < need <= tm._binding.NOALLOC_SCRATCH_BYTES, need
        say(f"noalloc decode call {n}: k_lens={k_lens} Hq={hq} Hkv={hkv} page={page} workspace {need} B")
        ref = run_gpu_decode(inp)
        q, kc, vc = inp["q"].to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev)
        sinks = inp["sinks"].to(dev)
        lens, table = inp["seqlens_k"].to(dev), inp["block_table"].to(dev)
        out = torch.full_like(q, float("nan"))
        got = tm.ts_mha_decode_with_kvcache_noalloc(q, kc, vc, sinks, lens, table, window=w,
                                                    softmax_scale=wl.softmax_scale, out=out,
                                                    max_seqlen_k=wl.max_seqlen_k)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.cpu().view(torch.int16), ref.cpu().view(torch.int16)), f"call {n}"
        oref = oracle.cache_attend(*cache_oracle_args(inp), lib=oracle_lib)
        excess = np.abs(f64(got.cpu()) - oref) - cache_rounding_bound(inp, oref, oracle_lib)
        assert excess.max() <= 0, f"call {n}: rounding bound exceeded by {excess.max():.3e}"


def test_noalloc_decode_refuses_more_than_its_scratch():
    """A split whose partials exceed the scratch is refused on the host, before any device
    call (so this runs without a GPU too)."""
    B, hq, hkv, L = 2048, 64, 8, 1 << 20
    need = tm.ts_mha_decode_workspace_size(B, hq, hkv, 64, 0, L)
    assert need > tm._binding.NOALLOC_SCRATCH_BYTES
    FAKE = 0x10000
    say("noalloc decode over its scratch")
    rc = tm.lib().ts_mha_decode_with_kvcache_noalloc(FAKE, FAKE, FAKE, None, FAKE, FAKE, hq, hkv, 64, 0,
                                                     0.125, FAKE * 2, B, 1 << 16, 16, L // 16, L, None)
    assert rc == -10
