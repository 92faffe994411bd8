"""Regression pin: the oracle's stored answer for the tiny dense workload.

tests/golden/c1_tiny_dense_seed0.npz was written by tests/golden/make_golden.py,
which calls only the oracle. A mismatch means the input recipe or the oracle's
arithmetic changed; such a change must name the passage that justifies it.
"""

import os

import numpy as np

import oracle
from synthetic import WORKLOADS, workload_inputs
from tests.golden.make_golden import input_digest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_c1_golden():
    g = np.load(os.path.join(HERE, "c1_tiny_dense_seed0.npz"), allow_pickle=False)
    w = WORKLOADS["c1_tiny_dense"]
    inp = workload_inputs(w)
    assert str(g["digest"]) == input_digest(inp)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal, w.softmax_scale)
    np.testing.assert_allclose(o, g["o"], atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, g["lse"], atol=1e-13, rtol=0)
