"""Stored fixtures: the seeded varlen draw and the oracle's tiny-workload output.

Both files are written by tests/golden/make_golden.py, which calls only the
oracle and the seeded generators.
"""
import json
import os

import numpy as np

from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import oracle_args

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_varlen_lengths_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "varlen16_lengths.json")))
    got = workloads.varlen16_lengths(seed=fx["seed"], lo=fx["low"], hi=fx["high_inclusive"])
    assert list(got) == fx["lengths"]
    assert workloads.WORKLOADS["varlen16_window128"].seqlens == tuple(fx["lengths"])
    assert sum(fx["lengths"]) == 78367 and max(fx["lengths"]) == 7942


def test_tiny_oracle_fixture(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "tiny_oracle.json")))
    wl = workloads.WORKLOADS[fx["workload"]]
    out = oracle.prefill(*oracle_args(workloads.make_inputs(wl, seed=fx["seed"])), lib=oracle_lib)
    for t, h, d, val in fx["sample"]:
        assert out[t, h, d] == val
    assert np.isclose(out.sum(), fx["sum"], rtol=1e-13, atol=1e-13)
    assert np.isclose((out ** 2).sum(), fx["sum_sq"], rtol=1e-13)
