"""Pins for the fp64 attention oracle, none of which re-types its formula.

The pages print no attention output values and no worked example, so the oracle
is pinned by (1) a pure-Python brute force on tiny inputs, (2) torch's float64
scaled_dot_product_attention on the CPU (a library routine for the special case
sq == sk), (3) closed forms and invariants of softmax attention, and (4) the
bf16 input recipe. ``test_mutants_are_caught`` plants plausible mistakes in the
oracle (on the CPU) and checks that these pins catch each one.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.reference as oa
from synthetic import cu_seqlens, cu_seqlens_linspace, make_inputs, WORKLOADS


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _case(lens, h, d, dv=None, seed=0):
    dv = d if dv is None else dv
    cq, ck = cu_seqlens(lens)
    q = _rand((int(cq[-1]), h, d), seed)
    k = _rand((int(ck[-1]), h, d), seed + 1)
    v = _rand((int(ck[-1]), h, dv), seed + 2)
    return q, k, v, cq, ck


TINY_CASES = [
    # (per-doc (sq, sk), heads, d, dv, causal)
    (((5, 5),), 1, 3, 3, False),
    (((5, 5),), 2, 4, 4, True),
    (((3, 7),), 1, 5, 2, True),          # sq < sk: bottom-right causal
    (((7, 3),), 2, 2, 5, True),          # sq > sk: leading rows see nothing
    (((4, 6), (2, 2), (6, 4)), 2, 3, 3, True),
    (((4, 6), (2, 2), (6, 4)), 1, 5, 4, False),
    (((1, 1), (0, 3), (3, 0)), 1, 2, 2, False),   # empty docs
    (((1, 1), (0, 3), (3, 0)), 1, 2, 2, True),
]


@pytest.mark.parametrize("lens,h,d,dv,causal", TINY_CASES)
def test_matches_bruteforce(lens, h, d, dv, causal):
    q, k, v, cq, ck = _case(lens, h, d, dv, seed=len(lens) + d)
    tau = 0.7
    o, lse = oracle.attention(q, k, v, cq, ck, causal, tau, row_block=2)
    ob, lb = oracle.attention_bruteforce(q, k, v, cq, ck, causal, tau)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)
    assert np.all(lse[~fin] == -np.inf) and np.all(lb[~fin] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s,d", [(1, 8), (17, 16), (64, 64), (129, 128)])
def test_matches_torch_sdpa_float64(causal, s, d):
    h = 3
    q, k, v, cq, ck = _case(((s, s),), h, d, seed=s)
    tau = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = oracle.attention(q, k, v, cq, ck, causal, tau, row_block=37)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=tau)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)
    # LSE via torch.logsumexp over the masked score matrix (library reduction)
    s_t = tau * torch.einsum("hqd,hkd->hqk", tq[0], tk[0])
    if causal:
        s_t = s_t.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(s_t, dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-10)


def test_rows_of_p_sum_to_one():
    q, k, v, cq, ck = _case(((40, 50),), 1, 8, seed=3)
    s = oracle.scores(q[:, 0], k[:, 0], 0.9)
    for causal in (False, True):
        p, m, lse = oracle.softmax_rows(s, oracle.visible(np.arange(40), 40, 50, causal))
        assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
        assert np.all(p >= 0)
        if causal:
            vis = oracle.visible(np.arange(40), 40, 50, True)
            assert np.all(p[~vis] == 0)


def test_constant_v_gives_v():
    q, k, v, cq, ck = _case(((33, 33), (5, 9)), 2, 8, seed=4)
    row = _rand((2, 8), 5)
    v[:] = row[None, :, :]
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, cq, ck, causal, 0.5)
        np.testing.assert_allclose(o, np.broadcast_to(row[None], o.shape), atol=1e-13, rtol=0)


def test_single_visible_key_gives_that_row():
    # sk = 1: every row sees exactly one key
    q, k, v, cq, ck = _case(((6, 1),), 2, 4, seed=6)
    o, lse = oracle.attention(q, k, v, cq, ck, False, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v[0][None], o.shape), atol=0, rtol=0)
    # causal row 0 (sq == sk) sees key 0 only: O = V_0, LSE = tau * q0.k0
    q, k, v, cq, ck = _case(((9, 9),), 3, 4, seed=7)
    tau = 0.45
    o, lse = oracle.attention(q, k, v, cq, ck, True, tau)
    np.testing.assert_array_equal(o[0], v[0])
    tau32 = float(np.float32(tau))
    for hh in range(3):
        assert abs(lse[hh, 0] - tau32 * float(np.dot(q[0, hh], k[0, hh]))) <= 1e-15


def test_zero_query_gives_mean_and_log_count():
    q, k, v, cq, ck = _case(((12, 12),), 2, 4, seed=8)
    q[:] = 0.0
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, cq, ck, causal, 1.0)
        for i in range(12):
            n = i + 1 if causal else 12
            np.testing.assert_allclose(o[i], v[:n].mean(axis=0), atol=1e-14, rtol=0)
            np.testing.assert_allclose(lse[:, i], math.log(n), atol=1e-14, rtol=0)


def test_noncausal_permutation_invariance():
    q, k, v, cq, ck = _case(((16, 21),), 2, 8, seed=9)
    o, lse = oracle.attention(q, k, v, cq, ck, False, 0.35)
    perm = np.random.default_rng(0).permutation(21)
    o2, lse2 = oracle.attention(q, k[perm], v[perm], cq, ck, False, 0.35)
    np.testing.assert_allclose(o2, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-13, rtol=0)


def test_scale_invariance():
    q, k, v, cq, ck = _case(((10, 10),), 1, 6, seed=10)
    tau = 0.25   # exact in fp32 and in binary, so tau*Q is exact
    o1, l1 = oracle.attention(q, k, v, cq, ck, True, tau)
    o2, l2 = oracle.attention(q * tau, k, v, cq, ck, True, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-13, rtol=0)


def test_lse_shift_identity():
    # adding a to every visible score shifts LSE by a and leaves O unchanged:
    # append a constant feature to q and a matching all-ones feature to k
    q, k, v, cq, ck = _case(((11, 11),), 1, 4, seed=11)
    a = 1.75
    q2 = np.concatenate([q, np.full(q.shape[:2] + (1,), a)], axis=2)
    k2 = np.concatenate([k, np.ones(k.shape[:2] + (1,))], axis=2)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, cq, ck, causal, 1.0)
        o2, l2 = oracle.attention(q2, k2, v, cq, ck, causal, 1.0)
        np.testing.assert_allclose(o2, o1, atol=1e-13, rtol=0)
        np.testing.assert_allclose(l2, l1 + a, atol=1e-13, rtol=0)


def test_causal_ignores_future_keys_exactly():
    q, k, v, cq, ck = _case(((20, 20),), 2, 8, seed=12)
    o, lse = oracle.attention(q, k, v, cq, ck, True, 0.4)
    i = 7
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] += 3.0
    v2[i + 1:] -= 5.0
    o2, lse2 = oracle.attention(q, k2, v2, cq, ck, True, 0.4)
    assert np.array_equal(o2[:i + 1], o[:i + 1])
    assert np.array_equal(lse2[:, :i + 1], lse[:, :i + 1])
    assert not np.allclose(o2[i + 1:], o[i + 1:])


def test_document_isolation_and_varlen_equals_per_doc():
    lens = ((13, 13), (7, 7), (30, 30))
    q, k, v, cq, ck = _case(lens, 2, 8, seed=13)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, cq, ck, causal, 0.3)
        for b in range(3):
            a0, a1 = cq[b], cq[b + 1]
            ob, lb = oracle.attention(q[a0:a1], k[a0:a1], v[a0:a1], [0, a1 - a0], [0, a1 - a0],
                                      causal, 0.3)
            assert np.array_equal(ob, o[a0:a1])
            assert np.array_equal(lb, lse[:, a0:a1])
        # perturbing doc 2 leaves docs 0 and 1 unchanged
        k2 = k.copy()
        k2[cq[2]:] += 1.0
        o2, l2 = oracle.attention(q, k2, v, cq, ck, causal, 0.3)
        assert np.array_equal(o2[:cq[2]], o[:cq[2]])


def test_sampled_rows_match_full():
    lens = ((50, 50), (70, 70))
    q, k, v, cq, ck = _case(lens, 3, 8, seed=14)
    o, lse = oracle.attention(q, k, v, cq, ck, True, 0.3)
    samples = [(0, 0), (49, 2), (50, 1), (119, 0), (77, 2)]
    os_, ls = oracle.attention_sampled(q, k, v, cq, ck, True, 0.3, samples)
    for n, (t, hh) in enumerate(samples):
        np.testing.assert_allclose(os_[n], o[t, hh], atol=1e-14, rtol=0)
        np.testing.assert_allclose(ls[n], lse[hh, t], atol=1e-14, rtol=0)


def test_empty_rows():
    q, k, v, cq, ck = _case(((4, 2),), 1, 3, seed=15)
    o, lse = oracle.attention(q, k, v, cq, ck, True, 1.0)
    # rows 0 and 1 see keys j <= i - 2: none
    assert np.all(o[:2] == 0) and np.all(lse[0, :2] == -np.inf)
    assert np.all(np.isfinite(lse[0, 2:]))


def test_bf16_inputs_are_widened_exactly():
    inp = make_inputs(((9, 9),), 2, 16, seed=3)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, True, 0.25)
    qf = inp.q.double().numpy()
    assert np.array_equal(qf, inp.q.float().numpy().astype(np.float64))
    o2, _ = oracle.attention(qf, inp.k.double().numpy(), inp.v.double().numpy(), inp.cu_q,
                             inp.cu_k, True, 0.25)
    assert np.array_equal(o, o2)


def test_input_recipe():
    # round(linspace(0, total, docs + 1)) as in the FA4 benchmark script
    assert cu_seqlens_linspace(8192, 4).tolist() == [0, 2048, 4096, 6144, 8192]
    assert cu_seqlens_linspace(32768, 8).tolist() == list(range(0, 32769, 4096))
    assert cu_seqlens_linspace(32768, 1).tolist() == [0, 32768]
    w = WORKLOADS["c2_dense_2225"]
    assert w.total_q == 2225 and w.heads == 16 and w.head_dim == 128 and not w.causal
    assert abs(WORKLOADS["c4_varlen_causal_32k"].flops() - 1.0995116e12) < 1e6
    assert abs(WORKLOADS["c2_dense_2225"].flops() - 40.56e9) < 0.01e9
    inp = make_inputs(((5, 5),), 2, 8, seed=0)
    inp2 = make_inputs(((5, 5),), 2, 8, seed=0)
    assert torch.equal(inp.q, inp2.q) and torch.equal(inp.v, inp2.v)
    assert inp.q.dtype == torch.bfloat16


# ---------------------------------------------------------------------------
# Mutation check: each planted mistake must be caught by at least one pin.
# ---------------------------------------------------------------------------

def _pins_pass():
    try:
        for args in TINY_CASES:
            test_matches_bruteforce(*args)
        test_matches_torch_sdpa_float64(True, 17, 16)
        test_matches_torch_sdpa_float64(False, 17, 16)
        test_single_visible_key_gives_that_row()
        test_zero_query_gives_mean_and_log_count()
        test_rows_of_p_sum_to_one()
        test_empty_rows()
    except AssertionError:
        return False
    return True


def _mut_causal_off_by_one(rows, sq, sk, causal):
    cols = np.arange(sk)[None, :]
    if not causal:
        return np.ones((len(rows), sk), dtype=bool)
    return cols < (np.asarray(rows)[:, None] + (sk - sq))


def _mut_causal_top_left(rows, sq, sk, causal):
    cols = np.arange(sk)[None, :]
    if not causal:
        return np.ones((len(rows), sk), dtype=bool)
    return cols <= np.asarray(rows)[:, None]


def _mut_lse_drops_max(s, mask):
    p, m, lse = _orig_softmax(s, mask)
    return p, m, np.where(np.isfinite(m), lse - m, lse)


def _mut_no_max_subtraction_sign(s, mask):
    p, m, lse = _orig_softmax(s, mask)
    return p, m, np.where(np.isfinite(m), lse - 2 * m, lse)


def _mut_scale_squared(q, k, tau):
    return tau * tau * (q @ k.T)


def _mut_scale_dropped(q, k, tau):
    return q @ k.T


def _mut_scores_transposed(q, k, tau):
    # the score matrix taken in the wrong orientation: S^T where it is square,
    # the keys in reverse order otherwise
    s = tau * (q @ k.T)
    return s.T if s.shape[0] == s.shape[1] else s[:, ::-1]


def _mut_values_transposed(q, k, v, rows, sq, causal, tau):
    # O = P V with V's rows taken in reverse key order (an index mistake on the
    # second operand)
    return _orig_attention_rows(q, k, v[::-1], rows, sq, causal, tau)


_orig_softmax = oa.softmax_rows
_orig_attention_rows = oa.attention_rows


@pytest.mark.parametrize("target,mutant", [
    ("visible", _mut_causal_off_by_one),
    ("visible", _mut_causal_top_left),
    ("softmax_rows", _mut_lse_drops_max),
    ("softmax_rows", _mut_no_max_subtraction_sign),
    ("scores", _mut_scale_squared),
    ("scores", _mut_scale_dropped),
    ("scores", _mut_scores_transposed),
    ("attention_rows", _mut_values_transposed),
])
def test_mutants_are_caught(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(oa, target, mutant)
    assert not _pins_pass(), f"planted mistake in {target} was not caught"
