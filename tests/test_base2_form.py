"""The base-2 form of the prefill kernels' query operand (_util.base2_inputs), on the CPU.

The tight GPU checks compare the kernel with the oracle run on bf16(q * scale * log2 e)
with scale ln 2.  That must be the same attention as the original inputs up to the
query's rounding: far closer than any mistake in the form (a wrong constant, the scale
applied twice or not at all) would leave it.
"""
import numpy as np
import torch

from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import LN2, base2_inputs, oracle_args


def test_base2_form_is_the_same_attention(oracle_lib):
    wl = workloads.custom([200, 77], 16, 2, window=0, seed=31)
    inp = workloads.make_inputs(wl)
    b2 = base2_inputs(inp)
    assert b2 is not inp and b2["softmax_scale"] == LN2 and b2["q"].dtype == torch.bfloat16
    ref = oracle.prefill(*oracle_args(inp), lib=oracle_lib)
    alt = oracle.prefill(*oracle_args(b2), lib=oracle_lib)
    d = np.abs(ref - alt)
    # the query's rounding moves a logit by at most 2^-8 * c * sum_d |q_d k_d| (about
    # 0.04 in base 2 here): a few 1e-4 on average, 1e-2 at worst on short rows, whose
    # outputs are near 1; dropping log2 e or applying the scale twice moves them by ~1e-1
    assert d.max() < 1e-2 and d.mean() < 5e-4, (d.max(), d.mean())
    assert d.max() > 0  # the query was really rounded
    # wrong forms are far away
    wrong = dict(b2, softmax_scale=1.0)
    bad = np.abs(ref - oracle.prefill(*oracle_args(wrong), lib=oracle_lib))
    assert bad.mean() > 30 * d.mean()


def test_base2_form_exact_when_the_fold_is_exact(oracle_lib):
    """With scale ln 2 the folded constant is 1: q is unchanged and the forms agree exactly."""
    wl = workloads.custom([90], 8, 2, window=0, softmax_scale=LN2, seed=32)
    inp = workloads.make_inputs(wl)
    b2 = base2_inputs(inp)
    assert torch.equal(b2["q"].view(torch.int16), inp["q"].view(torch.int16))
    np.testing.assert_array_equal(oracle.prefill(*oracle_args(inp), lib=oracle_lib),
                                  oracle.prefill(*oracle_args(b2), lib=oracle_lib))
