"""Merge of partial attention results over disjoint key ranges (the oracle).

TEST INFRASTRUCTURE (see ``oracle/reference.py``): imported only by tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py``.

A query row whose keys are split into disjoint ranges s has, per range,
O_s = sum_{j in s} exp(S_j) V_j / sum_{j in s} exp(S_j) and
LSE_s = ln sum_{j in s} exp(S_j). The softmax over the union is recovered by
the same rescaling by exp of a maximum difference that the online softmax
applies tile by tile ("[BUG] Unexpected Slower Performance in C++ CuTe
(77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on Jetson Thor", Key
Observation 2, the softmax_step listings), applied once across ranges:
    LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
Ranges without a visible key (LSE_s = -inf) weigh nothing; a row without any
visible key gets O = 0 and LSE = -inf.
"""

from __future__ import annotations

import numpy as np


def merge_partials(o_parts, lse_parts):
    """o_parts [S, n, d], lse_parts [S, n] (natural log) -> (O [n, d], LSE [n]), fp64."""
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    m = l.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(l - m_safe[None, :])                 # exp(-inf) = 0 for empty parts
    den = w.sum(axis=0)
    out = np.einsum("sn,snd->nd", w, o) / np.where(empty, 1.0, den)[:, None]
    out = np.where(empty[:, None], 0.0, out)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, den)))
    return out, lse
