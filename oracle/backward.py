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


def _backward_one(qb, kb, vb, dob, sq, causal, tau, row_block):
    """Gradients for one (document, head): q/do [sq, d], k/v [sk, d] in fp64."""
    sk = kb.shape[0]
    dq = np.zeros_like(qb)
    dk = np.zeros_like(kb)
    dv = np.zeros_like(vb)
    for r0 in range(0, sq, row_block):
        r1 = min(sq, r0 + row_block)
        rows = np.arange(r0, r1)
        s = scores(qb[r0:r1], kb, tau)
        p, _, _ = softmax_rows(s, visible(rows, sq, sk, causal))
        dp = dob[r0:r1] @ vb.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dv += p.T @ dob[r0:r1]
        dq[r0:r1] = tau * (ds @ kb)
        dk += tau * (ds.T @ qb[r0:r1])
    return dq, dk, dv


def attention_backward(q, k, v, dout, cu_seqlens_q: Sequence[int], cu_seqlens_k: Sequence[int],
                       causal: bool, softmax_scale: float, row_block: int = DEFAULT_ROW_BLOCK,
                       heads: Optional[Iterable[int]] = None,
                       docs: Optional[Iterable[int]] = None):
    """Gradients of packed varlen attention.

    q, dout [total_q, h, d]; k, v [total_k, h, d]; any float dtype (widened
    exactly to fp64). Returns (dQ, dK, dV) fp64 in the shapes of q, k, v. Rows
    of documents or heads not selected (``heads``/``docs``) are NaN.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    tau = float(np.float32(softmax_scale))
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    head_list = range(q.shape[1]) if heads is None else list(heads)
    doc_list = range(len(cq) - 1) if docs is None else list(docs)
    for b in doc_list:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        for hh in head_list:
            g = _backward_one(_as_f64(q[q0:q1, hh, :]), _as_f64(k[k0:k1, hh, :]),
                              _as_f64(v[k0:k1, hh, :]), _as_f64(dout[q0:q1, hh, :]),
                              q1 - q0, causal, tau, row_block)
            dq[q0:q1, hh, :], dk[k0:k1, hh, :], dv[k0:k1, hh, :] = g
    return dq, dk, dv
