"""Plain fp64 CPU attention: the oracle for the FMHA forward pass.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product path.

What it computes. The pages describe the FMHA forward pass as tiled Q.K^T, an
online softmax in the exp2 domain with the softmax scale and the running row
maximum folded into one fused multiply-add, then P.V with fp32 accumulation
("[BUG] Unexpected Slower Performance in C++ CuTe (77_blackwell_fmha) vs Python
CuTe DSL (fmha.py) on Jetson Thor", Key Observation 2, the two softmax_step
listings; "Kernel Bottleneck Tuning", section 4, log-domain refactoring). The
online form, the exp2 base change and the folds are identities, so in exact
arithmetic the method reaches exactly plain softmax attention. This oracle is
that plain definition, written out directly and slowly:

  1. S = tau * Q K^T for one document and one head, materialised row by row in
     full (tau is the fp32 value of the softmax scale the kernel receives);
  2. causal masking inside each document: key j is visible to query i iff
     j <= i + (sk - sq) (bottom-right alignment; j <= i when sq == sk, which
     is the varlen causal case of "CuTe DSL 4.7/4.8 regression: FlashAttention-4
     SM100 forward kernel spills registers", Steps/Code to reproduce bug);
  3. a standard two-pass softmax: m_i = max_j S_ij, then
     P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i);
  4. O = P V and LSE_i = m_i + ln sum_j exp(S_ij - m_i) (natural log of the
     scaled scores);
  5. a row with no visible key has O_i = 0 and LSE_i = -inf.

Everything runs in float64 on numpy; inputs are the exact bf16 values widened.
Documents are given by int32 prefix arrays cu_seqlens_q / cu_seqlens_k over a
packed [total_tokens, heads, d] layout, as in the benchmark script of the
FlashAttention-4 spill issue.

Memory. A document-head S can be larger than memory allows (32768^2 fp64 is
8.6 GB), so rows are materialised in blocks of full rows; each row's softmax is
over its complete row, so this is the same result as materialising all of S.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

# Rows of S materialised at once per (document, head); only a memory bound.
DEFAULT_ROW_BLOCK = 1024


def scores(q: np.ndarray, k: np.ndarray, tau: float) -> np.ndarray:
    """S = tau * q k^T for q [sq, d], k [sk, d] (fp64)."""
    return tau * (q @ k.T)


def visible(rows: np.ndarray, sq: int, sk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), sk]: which keys each query row may attend to.

    Non-causal rows see all sk keys. Causal rows see keys j <= i + (sk - sq).
    """
    cols = np.arange(sk)[None, :]
    if not causal:
        return np.ones((len(rows), sk), dtype=bool)
    return cols <= (np.asarray(rows)[:, None] + (sk - sq))


def softmax_rows(s: np.ndarray, mask: np.ndarray):
    """Two-pass softmax of each row of s over its visible entries.

    Returns (P, m, lse) with P [r, sk], m [r] (row max, -inf for an empty row)
    and lse [r] = m + ln(sum exp(s - m)) (-inf for an empty row). Rows with no
    visible key get P = 0.
    """
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=1)
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, denom)[:, None])
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, denom)))
    return p, m, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   sq: int, causal: bool, tau: float):
    """Attention for selected query rows of one (document, head).

    q [len(rows), d] holds those rows' queries; k [sk, d], v [sk, dv] hold the
    document's keys and values; rows are the query indices within the document.
    Returns (O [len(rows), dv], LSE [len(rows)]).
    """
    sk = k.shape[0]
    s = scores(q, k, tau)
    p, _, lse = softmax_rows(s, visible(rows, sq, sk, causal))
    o = p @ v
    return o, lse


def _as_f64(x) -> np.ndarray:
    """Widen a tensor/array (bf16 torch tensors included) to float64 numpy."""
    if hasattr(x, "detach"):               # torch tensor (CPU); exact widening
        return x.detach().to(dtype=_torch_float64()).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _torch_float64():
    import torch
    return torch.float64


def attention(q, k, v, cu_seqlens_q: Sequence[int], cu_seqlens_k: Sequence[int],
              causal: bool, softmax_scale: float, row_block: int = DEFAULT_ROW_BLOCK,
              heads: Optional[Iterable[int]] = None, docs: Optional[Iterable[int]] = None):
    """Plain attention over a packed varlen batch.

    q [total_q, h, d], k [total_k, h, d], v [total_k, h, dv]; any float dtype
    (widened exactly to fp64). cu_seqlens_q/k are int prefix arrays of length
    batch + 1. Returns (O [total_q, h, dv] fp64, LSE [h, total_q] fp64). Rows
    of documents or heads not selected (``heads``/``docs``) are NaN.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    tau = float(np.float32(softmax_scale))
    total_q, h, _ = q.shape
    dv = v.shape[2]
    out = np.full((total_q, h, dv), np.nan)
    lse = np.full((h, total_q), np.nan)
    head_list = range(h) if heads is None else list(heads)
    doc_list = range(len(cq) - 1) if docs is None else list(docs)
    for b in doc_list:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        sq = q1 - q0
        for hh in head_list:
            # widen only this (document, head) slice to fp64 (exact for bf16 inputs)
            qb = _as_f64(q[q0:q1, hh, :])
            kb, vb = _as_f64(k[k0:k1, hh, :]), _as_f64(v[k0:k1, hh, :])
            for r0 in range(0, sq, row_block):
                r1 = min(sq, r0 + row_block)
                rows = np.arange(r0, r1)
                o, l = attention_rows(qb[r0:r1], kb, vb, rows, sq, causal, tau)
                out[q0 + r0:q0 + r1, hh, :] = o
                lse[hh, q0 + r0:q0 + r1] = l
    return out, lse


def attention_sampled(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool, softmax_scale: float,
                      samples):
    """Attention for individual (token, head) pairs of a packed varlen batch.

    ``samples`` is an iterable of (global query token index, head). Returns
    (O [n, dv] fp64, LSE [n] fp64) in the order given. Each sample is computed
    from its complete score row, exactly as in ``attention``.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    tau = float(np.float32(softmax_scale))
    samples = list(samples)
    dv = v.shape[2]
    out = np.zeros((len(samples), dv))
    lse = np.zeros(len(samples))
    # group by (doc, head) so each K/V slice is widened once
    groups = {}
    for n, (t, hh) in enumerate(samples):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        groups.setdefault((b, int(hh)), []).append((n, int(t)))
    for (b, hh), items in groups.items():
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        kb = _as_f64(k[k0:k1, hh, :])
        vb = _as_f64(v[k0:k1, hh, :])
        idx = np.array([t for _, t in items])
        qb = _as_f64(q[idx.tolist(), hh, :])
        o, l = attention_rows(qb, kb, vb, idx - q0, q1 - q0, causal, tau)
        for j, (n, _) in enumerate(items):
            out[n] = o[j]
            lse[n] = l[j]
    return out, lse


def attention_bruteforce(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool,
                         softmax_scale: float):
    """Pure-Python loops with math.exp / math.fsum; for tiny inputs only.

    Same contract as ``attention`` but written element by element from the
    definition, so that it can pin the vectorised oracle on small cases.
    """
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    tau = float(np.float32(softmax_scale))
    total_q, h, d = qf.shape
    dv = vf.shape[2]
    out = [[[0.0] * dv for _ in range(h)] for _ in range(total_q)]
    lse = [[0.0] * total_q for _ in range(h)]
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        for hh in range(h):
            for i in range(sq):
                vis = [j for j in range(sk) if (not causal) or j <= i + sk - sq]
                if not vis:
                    lse[hh][q0 + i] = -math.inf
                    continue
                srow = {j: tau * math.fsum(float(qf[q0 + i, hh, c]) * float(kf[k0 + j, hh, c])
                                           for c in range(d)) for j in vis}
                mx = max(srow.values())
                ex = {j: math.exp(srow[j] - mx) for j in vis}
                z = math.fsum(ex.values())
                for c in range(dv):
                    out[q0 + i][hh][c] = math.fsum(ex[j] / z * float(vf[k0 + j, hh, c]) for j in vis)
                lse[hh][q0 + i] = mx + math.log(z)
    return np.array(out, dtype=np.float64).reshape(total_q, h, dv), np.array(lse, dtype=np.float64)
