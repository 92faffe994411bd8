"""Plain fp64 CPU gradients of attention: the oracle for the backward pass.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; it imports
nothing from the product path.

What it computes. The step the FlashAttention-4 spill issue times is a varlen
causal forward followed by the backward of the loss mean(O^2) ("CuTe DSL
4.7/4.8 regression: FlashAttention-4 SM100 forward kernel spills registers",
Describe the bug and the script under Steps/Code to reproduce bug); the pages
give no formula for that backward, so this module is the derivative of the
forward oracle's function, written out from the chain rule. For one document
and head with S = tau Q K^T (masked keys at -inf), P = softmax(S) row by row
and O = P V, and an upstream gradient dO:

  dV = P^T dO
  dP = dO V^T
  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)     (the softmax Jacobian of row i)
  dQ = tau dS K
  dK = tau dS^T Q

A query row with no visible key has P = 0 and contributes nothing; keys that
no query sees get dK = dV = 0. Everything is materialised in full rows of S in
float64 (rows in blocks, each row complete, as in the forward oracle).

Pins (tests/test_oracle_backward.py): central finite differences of the forward
oracle's sum(dO * O), invariants of the definition (the key gradients of a row
sum to zero, sum_j dV_j = sum_i dO_i over rows that see a key, constant V gives
dQ = dK = 0, a shift of all keys by one vector changes no gradient) and torch
float64 autograd through a plainly written dense attention.

Rounding scale (``rounding_scale=True``). The pages fix no precision for the
backward; the reading taken is the forward's: bf16 operands of every matrix
product, fp32 accumulation. A gradient element is then a sum whose terms carry
one bf16 rounding each (relative at most 2^-9): P's in dV_jd = sum_i P_ij dO_id,
dS's in dQ and dK, and the row value D_i = dO_i . O_i taken from a bf16 O, whose
error moves every dS_ij of row i by -P_ij dD_i. The scale returned per element
is the root sum of squares of those worst-case term errors,

  T(dV_jd) = 2^-9 sqrt(sum_i P_ij^2 dO_id^2)
  T(dQ_id) = tau sqrt(2^-18 sum_j dS_ij^2 K_jd^2 + e_i^2 (P K)_id^2)
  T(dK_jd) = tau sqrt(2^-18 sum_i dS_ij^2 Q_id^2 + sum_i P_ij^2 e_i^2 Q_id^2)

with e_i = sqrt(sum_d dO_id^2 o_id^2) and o_id = 2^-9 (|O_id| + sqrt(sum_j
P_ij^2 V_jd^2)) the size of O's own error (its final rounding and the bf16 P of
the forward's P.V). Independent unbiased roundings sum to an error of that
order; a parity bar is a multiple of it (plus the output's own rounding).
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .reference import DEFAULT_ROW_BLOCK, _as_f64, scores, softmax_rows, visible


def loss_grad_mean_square(o) -> np.ndarray:
    """dL/dO for L = mean(O^2) taken over all n elements of O: 2 O / n (fp64).

    This is the loss of the benchmark step in the FlashAttention-4 spill issue
    (the output, widened to fp32, squared and averaged, then backpropagated).
    """
    of = _as_f64(o)
    return 2.0 * of / of.size


_U = 2.0 ** -9   # unit roundoff of bf16 (round to nearest)


def _backward_one(qb, kb, vb, dob, sq, causal, tau, row_block, want_scale=False, first_row=0):
    """Gradients for one (document, head): q/do [sq, d], k/v [sk, d] in fp64.

    With want_scale, also the rounding scales T(dQ), T(dK), T(dV) (module
    docstring); their squares are accumulated over row blocks. Rows before
    ``first_row`` are skipped (see attention_backward)."""
    sk = kb.shape[0]
    dq = np.zeros_like(qb)
    dk = np.zeros_like(kb)
    dv = np.zeros_like(vb)
    t2q = np.zeros_like(qb)
    t2k = np.zeros_like(kb)
    t2v = np.zeros_like(vb)
    for r0 in range(first_row, sq, row_block):
        r1 = min(sq, r0 + row_block)
        rows = np.arange(r0, r1)
        s = scores(qb[r0:r1], kb, tau)
        p, _, _ = softmax_rows(s, visible(rows, sq, sk, causal))
        dp = dob[r0:r1] @ vb.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dv += p.T @ dob[r0:r1]
        dq[r0:r1] = tau * (ds @ kb)
        dk += tau * (ds.T @ qb[r0:r1])
        if want_scale:
            p2, ds2 = p * p, ds * ds
            o = p @ vb
            o_err = _U * (np.abs(o) + np.sqrt(p2 @ (vb * vb)))
            e2 = ((dob[r0:r1] * o_err) ** 2).sum(axis=1)          # e_i^2
            q2 = qb[r0:r1] ** 2
            t2v += _U * _U * (p2.T @ (dob[r0:r1] ** 2))
            t2q[r0:r1] = tau * tau * (_U * _U * (ds2 @ (kb * kb)) + e2[:, None] * (p @ kb) ** 2)
            t2k += tau * tau * (_U * _U * (ds2.T @ q2) + (p2 * e2[:, None]).T @ q2)
    if first_row > 0:
        # the skipped rows' dQ is unknown, and so are dK, dV of every key one of
        # them sees (causal: keys up to first_row - 1 + sk - sq; otherwise all)
        last_seen = first_row - 1 + (sk - sq) if causal else sk - 1
        for x in (dq, t2q):
            x[:first_row] = np.nan
        for x in (dk, dv, t2k, t2v):
            x[:max(0, last_seen + 1)] = np.nan
    if want_scale:
        return dq, dk, dv, np.sqrt(t2q), np.sqrt(t2k), np.sqrt(t2v)
    return dq, dk, dv


def attention_backward(q, k, v, dout, cu_seqlens_q: Sequence[int], cu_seqlens_k: Sequence[int],
                       causal: bool, softmax_scale: float, row_block: int = DEFAULT_ROW_BLOCK,
                       heads: Optional[Iterable[int]] = None,
                       docs: Optional[Iterable[int]] = None, rounding_scale: bool = False,
                       first_row: int = 0):
    """Gradients of packed varlen attention.

    q, dout [total_q, h, d]; k, v [total_k, h, d]; any float dtype (widened
    exactly to fp64). Returns (dQ, dK, dV) fp64 in the shapes of q, k, v, and
    with ``rounding_scale`` also their rounding scales (T(dQ), T(dK), T(dV)).
    Rows of documents or heads not selected (``heads``/``docs``) are NaN.
    ``first_row`` skips each document's first query rows (only the cost of a
    long document): their dQ, and dK and dV of every key they see, are NaN;
    everything else is exactly what the full computation gives.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    tau = float(np.float32(softmax_scale))
    outs = [np.full(x.shape, np.nan) for x in (q, k, v) * (2 if rounding_scale else 1)]
    head_list = range(q.shape[1]) if heads is None else list(heads)
    doc_list = range(len(cq) - 1) if docs is None else list(docs)
    for b in doc_list:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        for hh in head_list:
            g = _backward_one(_as_f64(q[q0:q1, hh, :]), _as_f64(k[k0:k1, hh, :]),
                              _as_f64(v[k0:k1, hh, :]), _as_f64(dout[q0:q1, hh, :]),
                              q1 - q0, causal, tau, row_block, rounding_scale,
                              min(first_row, q1 - q0))
            for n, x in enumerate(g):
                rows = slice(q0, q1) if n % 3 == 0 else slice(k0, k1)
                outs[n][rows, hh, :] = x
    if rounding_scale:
        return tuple(outs[:3]), tuple(outs[3:])
    return tuple(outs)
