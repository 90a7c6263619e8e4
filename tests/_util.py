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
