"""Pins for the oracle's merge of partial attention over disjoint key ranges."""

import numpy as np
import pytest

import oracle
from synthetic import make_inputs


def _partials(inp, causal, scale, cuts):
    """Per key range [cuts[r], cuts[r+1]) of every document: (O_r, LSE_r) for all
    (token, head) rows, from the oracle's scores and masked softmax."""
    tau = float(np.float32(scale))
    tq, h, d = inp.q.shape
    n_parts = len(cuts) - 1
    o = np.zeros((n_parts, tq, h, d))
    lse = np.full((n_parts, h, tq), -np.inf)
    for b in range(len(inp.cu_q) - 1):
        q0, q1 = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        k0, k1 = int(inp.cu_k[b]), int(inp.cu_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        for hh in range(h):
            qb = inp.q[q0:q1, hh].double().numpy()
            kb = inp.k[k0:k1, hh].double().numpy()
            vb = inp.v[k0:k1, hh].double().numpy()
            s = oracle.scores(qb, kb, tau)
            vis = oracle.visible(np.arange(sq), sq, sk, causal)
            for r in range(n_parts):
                lo, hi = int(cuts[r] * sk), int(cuts[r + 1] * sk)
                in_range = np.zeros(sk, dtype=bool)
                in_range[lo:hi] = True
                p, _, l = oracle.softmax_rows(s, vis & in_range[None, :])
                o[r, q0:q1, hh] = p @ vb
                lse[r, hh, q0:q1] = l
    return o, lse


@pytest.mark.parametrize("lens,causal,cuts", [
    (((40, 40),), False, [0, 0.5, 1]),
    (((40, 40), (17, 30)), True, [0, 0.3, 0.6, 1]),
    (((25, 60), (60, 25)), True, [0, 0.1, 0.2, 0.9, 1]),
    (((9, 9), (0, 5), (5, 0)), False, [0, 0.5, 1]),
    (((12, 12),), True, [0, 1.0, 1.0, 1.0]),          # empty trailing ranges
])
def test_merge_of_key_ranges_is_attention_over_all_keys(lens, causal, cuts):
    inp = make_inputs(lens, 2, 16, seed=3)
    scale = 0.3
    o_parts, lse_parts = _partials(inp, causal, scale, cuts)
    tq, h, d = inp.q.shape
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
    # rows (token, head) in token-major order
    o_m, lse_m = oracle.merge_partials(o_parts.reshape(len(cuts) - 1, tq * h, d),
                                       lse_parts.transpose(0, 2, 1).reshape(len(cuts) - 1, tq * h))
    assert np.allclose(o_m.reshape(tq, h, d), o_ref, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lse_ref.T.reshape(-1))
    assert np.array_equal(fin, np.isfinite(lse_m))
    assert np.allclose(lse_m[fin], lse_ref.T.reshape(-1)[fin], rtol=0, atol=1e-12)


def test_merge_special_cases():
    o = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])
    # equal LSEs average the parts; LSE grows by ln 2
    out, lse = oracle.merge_partials(o, np.array([[0.5], [0.5]]))
    assert np.allclose(out, [[2.0, 3.0]]) and np.allclose(lse, [0.5 + np.log(2.0)])
    # an empty part weighs nothing
    out, lse = oracle.merge_partials(o, np.array([[-np.inf], [1.25]]))
    assert np.array_equal(out, [[3.0, 4.0]]) and lse[0] == 1.25
    # nothing anywhere
    out, lse = oracle.merge_partials(o, np.array([[-np.inf], [-np.inf]]))
    assert np.array_equal(out, [[0.0, 0.0]]) and lse[0] == -np.inf
