"""Writes the stored fixtures under tests/golden/.  Calls only oracle/ (and the
seeded input generators); nothing here comes from the HIP path.

  varlen16_lengths.json  the seeded length draw of the 16-sequence varlen workload
                         (lengths uniform in [128, 8192], seed 1), an input fixture.
  tiny_oracle.json       oracle output of the 1 x 128, 4-over-1-head workload (seed 0)
                         at fixed sample positions, plus whole-array digests; it
                         guards the oracle and the generator against silent drift.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

from oracle import oracle  # noqa: E402
from sinks_ts_mha_amd import workloads  # noqa: E402
from _util import oracle_args  # noqa: E402

SAMPLE = [(0, 0, 0), (0, 3, 63), (1, 1, 7), (17, 2, 33), (64, 0, 1), (127, 3, 0), (127, 0, 63),
          (100, 1, 50), (31, 2, 31), (63, 3, 62)]


def tiny_fixture():
    wl = workloads.WORKLOADS["tiny_1x128_gqa4"]
    out = oracle.prefill(*oracle_args(workloads.make_inputs(wl)))
    return {
        "workload": wl.name,
        "seed": wl.seed,
        "sample": [[t, h, d, float(out[t, h, d])] for t, h, d in SAMPLE],
        "sum": float(out.sum()),
        "sum_sq": float((out ** 2).sum()),
    }


def main():
    with open(os.path.join(HERE, "varlen16_lengths.json"), "w") as f:
        json.dump({"seed": 1, "low": 128, "high_inclusive": 8192,
                   "lengths": list(workloads.varlen16_lengths())}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(tiny_fixture(), f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
