"""Pins of the backward oracle (oracle.attention_backward) to things other than itself.

* Central finite differences of the forward oracle: for L = sum(dO * O(q, k, v))
  the gradient of L in every input element must match the oracle's dQ, dK, dV.
  The forward oracle is pinned on its own (tests/test_oracle.py), and a dropped
  term, a wrong sign or a transposed operand anywhere in the backward fails here.
* Invariants of the definition: each row's score gradients sum to zero, so
  sum_j dK_j = 0; P's rows sum to one, so sum_j dV_j = sum_i dO_i over the rows
  that see a key; O does not depend on Q or K when V is constant, nor on a shift
  of all keys by one vector; the gradients are linear in dO.
* torch float64 autograd through a plainly written dense attention.
* The rounding scale (the parity bar's unit) against an emulation of the bf16
  operand roundings it models, which it must cover, and a planted masking
  mistake, which must exceed the bar.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_dout, make_inputs

LENS = ((5, 5), (3, 7), (6, 2), (0, 3), (4, 0), (1, 1))


def _tiny(lens, h, d, seed):
    rng = np.random.default_rng(seed)
    tq = sum(a for a, _ in lens)
    tk = sum(b for _, b in lens)
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int64)
    q = rng.standard_normal((tq, h, d))
    k = rng.standard_normal((tk, h, d))
    v = rng.standard_normal((tk, h, d))
    do = rng.standard_normal((tq, h, d))
    return q, k, v, do, cu_q, cu_k


def _loss(q, k, v, do, cu_q, cu_k, causal, scale):
    o, _ = oracle.attention(q, k, v, cu_q, cu_k, causal, scale)
    return float((do * o).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    q, k, v, do, cu_q, cu_k = _tiny(LENS, 2, 4, seed=1)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu_q, cu_k, causal, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(q, k, v, do, cu_q, cu_k, causal, scale)
            x[idx] = keep - eps
            lm = _loss(q, k, v, do, cu_q, cu_k, causal, scale)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - g).max() < 1e-7, (name, np.abs(num - g).max())


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    q, k, v, do, cu_q, cu_k = _tiny(((9, 9), (4, 11), (12, 5)), 3, 8, seed=2)
    scale = 0.5
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu_q, cu_k, causal, scale)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sq, sk = q1 - q0, k1 - k0
        seen = np.arange(sq) + (sk - sq) >= 0 if causal else np.ones(sq, bool)
        # score gradients of a row sum to zero
        assert np.abs(dk[k0:k1].sum(axis=0)).max() < 1e-12
        # P's rows sum to one over the rows that see a key
        np.testing.assert_allclose(dv[k0:k1].sum(axis=0), do[q0:q1][seen].sum(axis=0),
                                   atol=1e-12)
        # rows that see no key have no gradient
        assert np.all(dq[q0:q1][~seen] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_and_key_shift(causal):
    q, k, v, do, cu_q, cu_k = _tiny(((7, 7), (5, 9)), 2, 6, seed=3)
    scale = 0.9
    # constant V within each (document, head): O is V's row whatever Q and K are
    vc = v.copy()
    for b in range(len(cu_k) - 1):
        vc[cu_k[b]:cu_k[b + 1]] = v[cu_k[b]]
    dq, dk, _ = oracle.attention_backward(q, k, vc, do, cu_q, cu_k, causal, scale)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # a shift of every key of a (document, head) by one vector adds a constant
    # to each score row, which softmax ignores
    g0 = oracle.attention_backward(q, k, v, do, cu_q, cu_k, causal, scale)
    ks = k.copy()
    rng = np.random.default_rng(4)
    for b in range(len(cu_k) - 1):
        ks[cu_k[b]:cu_k[b + 1]] += rng.standard_normal((1,) + k.shape[1:])
    g1 = oracle.attention_backward(q, ks, v, do, cu_q, cu_k, causal, scale)
    for a, b_ in zip(g0, g1):
        np.testing.assert_allclose(a, b_, atol=1e-11)


def test_linear_in_dout_and_row_blocks():
    q, k, v, do, cu_q, cu_k = _tiny(((13, 13), (6, 10)), 2, 8, seed=5)
    do2 = np.random.default_rng(6).standard_normal(do.shape)
    g1 = oracle.attention_backward(q, k, v, do, cu_q, cu_k, True, 0.4)
    g2 = oracle.attention_backward(q, k, v, do2, cu_q, cu_k, True, 0.4)
    g3 = oracle.attention_backward(q, k, v, do + 2 * do2, cu_q, cu_k, True, 0.4, row_block=3)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(a + 2 * b, c, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_dense(causal):
    """Dense equal-length documents, against torch float64 autograd."""
    b, s, h, d = 2, 11, 3, 16
    q, k, v, do, cu_q, cu_k = _tiny(((s, s),) * b, h, d, seed=7)
    scale = 1 / np.sqrt(d)
    tau = float(np.float32(scale))
    qt, kt, vt = (torch.from_numpy(x.reshape(b, s, h, d)).permute(0, 2, 1, 3).clone()
                  .requires_grad_(True) for x in (q, k, v))
    st = tau * (qt @ kt.transpose(-1, -2).contiguous())
    if causal:
        st = st.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), float("-inf"))
    ot = torch.softmax(st, dim=-1) @ vt
    ot.backward(torch.from_numpy(do.reshape(b, s, h, d)).permute(0, 2, 1, 3))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu_q, cu_k, causal, scale)
    for g, t in ((dq, qt), (dk, kt), (dv, vt)):
        ref = t.grad.permute(0, 2, 1, 3).reshape(b * s, h, d).numpy()
        np.testing.assert_allclose(g, ref, atol=1e-12)


def test_mean_square_loss_gradient():
    o = torch.randn(5, 3, 4, dtype=torch.float64, requires_grad=True)
    o.square().mean().backward()
    np.testing.assert_allclose(oracle.loss_grad_mean_square(o.detach()), o.grad.numpy(),
                               atol=1e-15)


def _bf16(x):
    return (torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()
            .astype(np.float64))


def _emulated_bf16_backward(q, k, v, do, cu_q, cu_k, causal, tau, drop_key=None):
    """The backward with the roundings the rounding scale models: the forward's O
    from a bf16 P and rounded to bf16, D from that O, P and dS rounded to bf16 as
    operands, outputs rounded to bf16. drop_key=(doc, j) hides key j of that
    document from every row (a planted masking mistake)."""
    out = [np.zeros_like(x) for x in (q, k, v)]
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sq, sk = q1 - q0, k1 - k0
        vis = oracle.visible(np.arange(sq), sq, sk, causal)
        if drop_key is not None and drop_key[0] == b:
            vis = vis.copy()
            vis[:, drop_key[1]] = False
        for h in range(q.shape[1]):
            p, _, _ = oracle.softmax_rows(tau * q[q0:q1, h] @ k[k0:k1, h].T, vis)
            o = _bf16(_bf16(p) @ v[k0:k1, h])
            dp = do[q0:q1, h] @ v[k0:k1, h].T
            dsb = _bf16(p * (dp - (do[q0:q1, h] * o).sum(1)[:, None]))
            out[0][q0:q1, h] = _bf16(tau * dsb @ k[k0:k1, h])
            out[1][k0:k1, h] = _bf16(tau * dsb.T @ q[q0:q1, h])
            out[2][k0:k1, h] = _bf16(_bf16(p).T @ do[q0:q1, h])
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_rounding_scale_covers_bf16_operands(causal):
    """The rounding scale bounds the error of bf16 operands: an emulation of those
    roundings stays within 6 T + 2^-8 |g| (the GPU bar is 8 T + 2^-8 |g|), and a
    planted mistake (one key hidden from every row) does not."""
    lens = ((200, 200), (70, 150), (129, 129))
    q, k, v, do, cu_q, cu_k = _tiny(lens, 2, 64, seed=11)
    q, k, v, do = (_bf16(x) for x in (q, k, v, do))
    tau = float(np.float32(1 / 8))
    ref, scale = oracle.attention_backward(q, k, v, do, cu_q, cu_k, causal, tau,
                                           rounding_scale=True)
    emu = _emulated_bf16_backward(q, k, v, do, cu_q, cu_k, causal, tau)
    for e, r, t in zip(emu, ref, scale):
        assert np.all(np.abs(e - r) <= 6 * t + 2.0 ** -8 * np.abs(r))
    bad = _emulated_bf16_backward(q, k, v, do, cu_q, cu_k, causal, tau, drop_key=(0, 37))
    assert any(np.any(np.abs(e - r) > 8 * t + 2.0 ** -8 * np.abs(r))
               for e, r, t in zip(bad, ref, scale))
    # the scale is a small fraction of the gradients' size, not a blanket allowance
    for r, t in zip(ref, scale):
        assert np.median(t) < 5e-3 * np.sqrt(np.mean(r * r))


def test_skipping_first_rows_leaves_the_rest_exact():
    """first_row only drops work: every gradient it still reports equals the full
    computation's (up to the summation order of its row blocks), and the ones it
    cannot know are NaN."""
    inp = make_inputs(((70, 70), (50, 60)), 2, 16, seed=8)
    dout = make_dout(inp.q.shape[0], 2, 16, seed=8)
    for causal in (False, True):
        full = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, causal,
                                         0.25, row_block=16)
        part = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, causal,
                                         0.25, row_block=16, first_row=33)
        for f, g in zip(full, part):
            known = ~np.isnan(g)
            assert np.allclose(f[known], g[known], rtol=1e-12, atol=1e-15)
        dq, dk, _ = part
        assert np.isnan(dq[:33]).all() and not np.isnan(dq[33:70]).any()
        if causal:    # doc 0: keys 33..69 are seen only by rows >= 33
            assert np.isnan(dk[:33]).all() and not np.isnan(dk[33:70]).any()
            # doc 1 (sq 50, sk 60): rows >= 33 alone see keys >= 43
            assert np.isnan(dk[70:70 + 43]).all() and not np.isnan(dk[70 + 43:]).any()
        else:
            assert np.isnan(dk).all()


# ---------------------------------------------------------------------------
# Mutation check: planted mistakes in a copy of the oracle's per-head
# backward must each fail a pin above.
# ---------------------------------------------------------------------------

def _pins_pass():
    try:
        for causal in (False, True):
            test_finite_differences(causal)
            test_invariants(causal)
            test_torch_autograd_dense(causal)
    except AssertionError:
        return False
    return True


_MUTATIONS = {
    # dS = P * dP: the softmax Jacobian's row term dropped
    "dropped_jacobian_term": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                              "ds = p * dp"),
    # dK = tau dS^T Q with dS^T's rows taken in the wrong (reversed) key order
    "transposed_dk": ("dk += tau * (ds.T @ qb[r0:r1])", "dk += tau * (ds.T[::-1] @ qb[r0:r1])"),
    # dV from P without the transpose, reading keys in reverse order
    "dv_wrong_orientation": ("dv += p.T @ dob[r0:r1]", "dv += p.T[::-1] @ dob[r0:r1]"),
    # dQ without the softmax scale
    "dq_scale_dropped": ("dq[r0:r1] = tau * (ds @ kb)", "dq[r0:r1] = ds @ kb"),
}


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_backward_mutants_are_caught(monkeypatch, name):
    import inspect
    from oracle import backward as ob
    assert _pins_pass()
    old, new = _MUTATIONS[name]
    src = inspect.getsource(ob._backward_one)
    assert old in src, f"mutation site for {name} not found"
    ns = dict(vars(ob))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(ob, "_backward_one", ns["_backward_one"])
    assert not _pins_pass(), f"planted mistake {name} was not caught"
