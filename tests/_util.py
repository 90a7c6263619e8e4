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


LN2 = 0.6931471805599453


def base2_inputs(inp: dict) -> dict:
    """The attention the prefill kernels evaluate, as oracle inputs.

    The prefill kernels fold softmax_scale * log2(e) into their query operand:
    q~ = bf16(fp32(q) * c) with c = fp32(scale * log2 e), each step rounded to
    nearest even, and take exp2 of q~.k.  exp2(q~.k) is exp(ln2 * q~.k), so the
    oracle run on q~ with scale ln 2 (sinks unchanged: they stay natural-log
    logits) is exactly that attention; what remains between it and the kernel
    are the roundings rounding_bound covers.  Works on packed (make_inputs) and
    cache (make_cache_inputs) input dicts.
    """
    scale = float(np.float32(inp["softmax_scale"]))
    c = np.float32(scale * 1.4426950408889634)
    qt = (inp["q"].to(torch.float32) * torch.tensor(c, dtype=torch.float32)).to(torch.bfloat16)
    return dict(inp, q=qt, softmax_scale=LN2)


GATE_MAX, GATE_MEAN = 2e-2, 2e-3


def assert_within_rounding(got, inp: dict, lib=None, gate: bool = True, what: str = ""):
    """got (fp64) within rounding_bound of the oracle on the attention the kernel
    evaluates (base2_inputs); with gate, also within the parity gate (max |err| <=
    2e-2, mean <= 2e-3) of the oracle on the original inputs."""
    from oracle import oracle
    b2 = base2_inputs(inp)
    ref2 = oracle.prefill(*oracle_args(b2), lib=lib)
    excess = np.abs(got - ref2) - rounding_bound(b2, ref2, lib)
    assert excess.max() <= 0, f"{what}: rounding bound exceeded by {excess.max():.3e}"
    if gate:
        ref = oracle.prefill(*oracle_args(inp), lib=lib)
        d = np.abs(got - ref)
        assert d.max() <= GATE_MAX and d.mean() <= GATE_MEAN, \
            f"{what}: gate max {d.max():.3e} mean {d.mean():.3e}"


def rounding_bound(inp: dict, ref, lib=None):
    """Elementwise error allowance of a bf16-P, fp32-accumulate, bf16-output kernel.

    bf16 keeps 8 significant bits, so round-to-nearest has unit roundoff
    u = 2^-8.  Rounding each probability to bf16 moves the weighted sum of
    output element d by at most u * sum_j p_j |v_jd| (p normalised, sink
    included).  The kernel's denominator is the sum of those same rounded
    probabilities plus the sink's term, which moves the normalisation by at
    most u relative, i.e. the output by u |out_d|; rounding the output to bf16
    adds another u |out_d|.  sum_j p_j |v_jd| is the oracle's output for |v|
    (bf16 |v| is exact).  fp32 accumulation adds relative terms near 2^-20,
    covered by a factor (1 + 2^-6) and an absolute 1e-6.
    """
    from oracle import oracle
    weighted_abs = oracle.prefill(*oracle_args(dict(inp, v=inp["v"].abs())), lib=lib)
    return 2.0 ** -8 * (1 + 2.0 ** -6) * (weighted_abs + 2.0 * np.abs(ref)) + 1e-6


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
    return 2.0 ** -8 * (1 + 2.0 ** -6) * (weighted_abs + 2.0 * np.abs(ref)) + 1e-6


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
