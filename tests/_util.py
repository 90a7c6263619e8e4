"""Helpers shared by the tests: tensor <-> numpy conversion and error statistics.

No attention arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch

from sinks_ts_mha_amd.workloads import bf16_bits


def oracle_args(inp: dict):
    """Arguments of oracle.prefill(...) for an input dict from workloads.make_inputs."""
    sinks = inp["sinks"]
    return (bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]),
            None if sinks is None else sinks.detach().cpu().numpy().astype(np.float32),
            inp["cu_seqlens"].cpu().numpy().astype(np.int32), inp["window"],
            inp["softmax_scale"])


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def err_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "ref_rms": float(np.sqrt((ref.astype(np.float64) ** 2).mean())) if ref.size else 0.0}


def run_gpu(inp: dict, out=None, stream=None, window=None) -> torch.Tensor:
    """Run the HIP path (through the C ABI) on an input dict; returns the GPU output tensor."""
    import sinks_ts_mha_amd as tm
    dev = torch.device("cuda", 0)
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    sinks = None if inp["sinks"] is None else inp["sinks"].to(dev)
    cu = inp["cu_seqlens"].to(dev)
    return tm.ts_mha_prefill(q, k, v, sinks, cu, window=inp["window"] if window is None else window,
                             softmax_scale=inp["softmax_scale"], out=out,
                             max_seqlen=inp["max_seqlen"], stream=stream)


def say(msg: str):
    """Name the case before a GPU step, flushed, so a crash report shows where it was."""
    print(f"[gpu-case] {msg}", flush=True)


GATE_MAX, GATE_MEAN = 2e-2, 2e-3


def max_visible_keys(inp: dict) -> int:
    """Most keys any query row of a packed input dict sees (its longest causal/window run)."""
    cu = inp["cu_seqlens"].tolist()
    L = max([cu[b + 1] - cu[b] for b in range(len(cu) - 1)] + [0])
    w = inp["window"]
    return min(L, w) if w > 0 else L


def accumulation_allowance(n_keys: int) -> float:
    """Relative error allowance of the kernels' fp32 accumulations over n_keys keys.

    The output and the row sums are accumulated on the matrix pipe, at least 16 keys
    per fp32 addition into the accumulator; a recursive fp32 sum of m nonnegative-weight
    terms is within (m - 1) 2^-24 of the sum of their magnitudes.  Sixteen more units
    cover the fp32 score (bf16 products are exact, each MFMA adds its 16 to the
    accumulator once), the product by scale * log2 e, exp2, the normalisation and the
    sink's term.  Never below 2^-14, the allowance the short-row tests were written
    with.
    """
    return max(2.0 ** -14, (-(-n_keys // 16) + 16) * 2.0 ** -24)


def assert_within_rounding(got, inp: dict, lib=None, what: str = ""):
    """got (fp64) within rounding_bound of the oracle on the same inputs, and within
    the parity gate (max |err| <= 2e-2, mean <= 2e-3)."""
    from oracle import oracle
    ref = oracle.prefill(*oracle_args(inp), lib=lib)
    excess = np.abs(got - ref) - rounding_bound(inp, ref, lib)
    assert excess.max() <= 0, f"{what}: rounding bound exceeded by {excess.max():.3e}"
    d = np.abs(got - ref)
    assert d.max() <= GATE_MAX and d.mean() <= GATE_MEAN, \
        f"{what}: gate max {d.max():.3e} mean {d.mean():.3e}"


def rounding_bound(inp: dict, ref, lib=None, rows=None, heads=None):
    """Elementwise error allowance of a bf16-P, fp32-accumulate, bf16-output kernel.

    bf16 keeps 8 significant bits, so round-to-nearest has unit roundoff
    u = 2^-8.  Rounding each probability to bf16 moves the weighted sum of
    output element d by at most u * sum_j p_j |v_jd| (p normalised, sink
    included).  The kernel's denominator is the sum of those same rounded
    probabilities plus the sink's term, which moves the normalisation by at
    most u relative, i.e. the output by u |out_d|; rounding the output to bf16
    adds another u |out_d|.  sum_j p_j |v_jd| is the oracle's output for |v|
    (bf16 |v| is exact).  The fp32 accumulations add accumulation_allowance
    relative to the same magnitudes, plus an absolute 1e-6.  With rows/heads,
    ref holds the oracle's rows [n, D] (oracle.prefill_rows) and so does the
    result.
    """
    from oracle import oracle
    absv = dict(inp, v=inp["v"].abs())
    if rows is None:
        weighted_abs = oracle.prefill(*oracle_args(absv), lib=lib)
    else:
        weighted_abs = oracle.prefill_rows(*oracle_args(absv), rows=rows, heads=heads, lib=lib)
    gamma = accumulation_allowance(max_visible_keys(inp))
    return (2.0 ** -8 + gamma) * (weighted_abs + 2.0 * np.abs(ref)) + 1e-6


def cache_oracle_args(inp: dict):
    """Arguments of oracle.cache_attend(...) for an input dict from workloads.make_cache_inputs."""
    sinks = inp["sinks"]
    return (bf16_bits(inp["q"]), bf16_bits(inp["k_cache"]), bf16_bits(inp["v_cache"]),
            None if sinks is None else sinks.detach().cpu().numpy().astype(np.float32),
            inp["cu_seqlens_q"].cpu().numpy().astype(np.int32),
            inp["seqlens_k"].cpu().numpy().astype(np.int32),
            inp["block_table"].cpu().numpy().astype(np.int32), inp["window"],
            inp["softmax_scale"])


def run_gpu_decode(inp: dict, out=None, stream=None, workspace=None, k_cache=None, v_cache=None):
    """Run the decode kernels (through the C ABI) on a cache input dict; returns the GPU output."""
    import sinks_ts_mha_amd as tm
    dev = torch.device("cuda", 0)
    kc = (inp["k_cache"] if k_cache is None else k_cache).to(dev)
    vc = (inp["v_cache"] if v_cache is None else v_cache).to(dev)
    sinks = None if inp["sinks"] is None else inp["sinks"].to(dev)
    return tm.ts_mha_decode_with_kvcache(
        inp["q"].to(dev), kc, vc, sinks, inp["seqlens_k"].to(dev), inp["block_table"].to(dev),
        window=inp["window"], softmax_scale=inp["softmax_scale"], out=out,
        max_seqlen_k=inp["max_seqlen_k"], workspace=workspace, stream=stream)


def cache_rounding_bound(inp: dict, ref, lib=None):
    """rounding_bound for the cache form: the same roundings (bf16 probabilities in the
    numerator, fp32 denominator or its bf16 image, bf16 output), with sum_j p_j |v_jd|
    from the oracle's cache form applied to |v|."""
    from oracle import oracle
    args = list(cache_oracle_args(inp))
    args[2] = bf16_bits(inp["v_cache"].abs())
    weighted_abs = oracle.cache_attend(*args, lib=lib)
    n_keys = int(inp["seqlens_k"].max()) if inp["seqlens_k"].numel() else 0
    if inp["window"] > 0:
        n_keys = min(n_keys, inp["window"])
    gamma = accumulation_allowance(n_keys)
    return (2.0 ** -8 + gamma) * (weighted_abs + 2.0 * np.abs(ref)) + 1e-6


def run_gpu_prefill_kv(inp: dict, out=None, stream=None, k_cache=None, v_cache=None):
    """Run the prefill against a paged cache (through the C ABI); returns the GPU output."""
    import sinks_ts_mha_amd as tm
    dev = torch.device("cuda", 0)
    kc = (inp["k_cache"] if k_cache is None else k_cache).to(dev)
    vc = (inp["v_cache"] if v_cache is None else v_cache).to(dev)
    sinks = None if inp["sinks"] is None else inp["sinks"].to(dev)
    return tm.ts_mha_prefill_with_kvcache(
        inp["q"].to(dev), kc, vc, sinks, inp["cu_seqlens_q"].to(dev), inp["seqlens_k"].to(dev),
        inp["block_table"].to(dev), window=inp["window"], softmax_scale=inp["softmax_scale"],
        out=out, max_seqlen_q=inp["max_seqlen_q"], max_seqlen_k=inp["max_seqlen_k"], stream=stream)
