"""OCP e2m1 (FP4) decoding/encoding and the fp4 P.V oracles.

TEST INFRASTRUCTURE (see ``oracle/reference.py``): imported only by tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py``.

The fp4 P.V variant ("Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
GB300)", introduction; section 4, log-domain refactoring) runs the second GEMM
with both P and V in 4-bit e2m1, each element carrying a power-of-two block
scale.

E2M1 (OCP 4-bit float): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
bit; exponent field 0 encodes the subnormal m/2; no infinity or NaN. The
non-negative values are 0, 0.5, 1, 1.5, 2, 3, 4, 6.

V (input format, MXFP4). V arrives as e2m1 codes, two per byte along head_dim
(even d in the low nibble), and one E8M0 exponent byte per block of 32
consecutive tokens of the packed tensor, per head and per d:
    V_hat[t, h, d] = e2m1(code[t, h, d]) * 2^(scale[t // 32, h, d] - 127).

P (the method's quantisation). With c = fp32(softmax_scale * log2 e) and raw
scores r_j = q.k_j, a *group* is the set of keys of one query row that lie in
one 32-token block. exp2 is monotonic, so the group's largest 2^(c r_j) is
2^(c g_G) with g_G the group's largest raw score, and its power-of-two scale is
read off in the log domain:
    E_G = ceil(c g_G - log2 6)       (so 2^(c r_j - E_G) <= 6 = e2m1's maximum)
    P_hat_j = 2^E_G * e2m1(2^(c r_j - E_G))   (round to nearest, ties to even)
The division by the group scale is the subtraction of E_G inside the exp2
argument, as section 4 of that page folds post-exp scales. The row sum keeps the
unquantised values, l_i = sum_j 2^(c r_j), so LSE stays exact, and
O_i = sum_j P_hat_j V_hat_j / l_i.

Two answers are computed:
  * ``attention_fp4pv``: exact attention of (Q, K, V_hat), the function the
    inputs define; the P quantisation is the method's approximation, bounded
    by ``FP4Emulation.bound``.
  * ``attention_fp4pv_emulated``: the method's quantised result, computed from
    the definition above in fp64 (c = tau log2 e and every E_G and rounding
    decided exactly), plus what is left ambiguous when the scores are fp32 (as
    on the GPU): an element whose scaled value lies closer to an e2m1 rounding
    midpoint, or a group whose E_G argument lies closer to an integer, than
    the fp32 evaluation can be trusted (``oracle.fp32_window``) may take the
    other branch. Either choice is a correct result of the method; the
    ``ambiguity`` term is how far the other choices move O, and it is zero for
    every element whose row has no such decision.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import fp32_window
from .reference import _as_f64, attention, attention_sampled, visible

E2M1_MAX = 6.0
MX_BLOCK = 32                 # tokens per V scale block and per P group
LOG2_6 = float(np.log2(6.0))


def _e2m1_value(c: int) -> float:
    """Value of one 4-bit e2m1 code, from the format definition."""
    sign = -1.0 if c & 0x8 else 1.0
    e, m = (c >> 1) & 0x3, c & 0x1
    if e == 0:
        return sign * m / 2.0                       # subnormal
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit e2m1 codes (low nibble of each integer) to float64."""
    return _E2M1_TABLE[np.asarray(codes).astype(np.intp) & 0xF]


_POS_CODES = np.arange(8, dtype=np.int64)


def e2m1_encode(x) -> np.ndarray:
    """Round float64 values to the nearest e2m1 code, ties to an even code.

    Magnitudes above 6 saturate to 6; the sign of zero is dropped. Exhaustive
    search over the 8 non-negative codes: slow but plainly correct.
    """
    x = np.asarray(x, dtype=np.float64)
    vals = e2m1_decode(_POS_CODES)
    a = np.minimum(np.abs(x), E2M1_MAX).reshape(-1)
    out = np.empty(a.shape, dtype=np.int64)
    chunk = 1 << 18
    even = (_POS_CODES & 1) == 0
    for s in range(0, a.size, chunk):
        seg = a[s:s + chunk]
        d = np.abs(seg[:, None] - vals[None, :])
        tie = d == d.min(axis=1, keepdims=True)
        pick = np.where((tie & even).any(axis=1), np.argmax(tie & even, axis=1),
                        np.argmax(tie, axis=1))
        out[s:s + chunk] = _POS_CODES[pick]
    out = out.reshape(x.shape)
    return np.where(np.signbit(x) & (out != 0), out | 0x8, out).astype(np.uint8)


def _e2m1_midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Relative distance of |x| (<= 6) to the nearest e2m1 rounding midpoint."""
    vals = e2m1_decode(_POS_CODES)
    mids = (vals[1:] + vals[:-1]) / 2.0
    a = np.abs(x)
    d = np.abs(a[..., None] - mids).min(axis=-1)
    return d / np.maximum(a, 1e-300)


def _e2m1_step(x: np.ndarray) -> np.ndarray:
    """Gap between the two e2m1 values around |x| (the cost of a flipped rounding)."""
    a = np.abs(x)
    return np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))


def unpack_e2m1(packed, head_dim: int) -> np.ndarray:
    """uint8 [..., head_dim/2] -> codes [..., head_dim]; even d in the low nibble."""
    b = packed.numpy() if hasattr(packed, "numpy") else np.asarray(packed)
    b = b.astype(np.uint8)
    assert b.shape[-1] * 2 == head_dim
    out = np.empty(b.shape[:-1] + (head_dim,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def mx_dequantize_v(v_packed, v_scales, head_dim: int) -> np.ndarray:
    """V_hat[t, h, d] = e2m1(code) * 2^(scale[t // 32, h, d] - 127), fp64."""
    codes = unpack_e2m1(v_packed, head_dim)
    sc = v_scales.numpy() if hasattr(v_scales, "numpy") else np.asarray(v_scales)
    t = codes.shape[0]
    blk = np.arange(t) // MX_BLOCK
    exps = sc.astype(np.int64)[blk] - 127
    return np.ldexp(e2m1_decode(codes), exps)


def attention_fp4pv(q, k, v_packed, v_scales, cu_seqlens_q, cu_seqlens_k, causal: bool,
                    softmax_scale: float, **kw):
    """Exact attention of (Q, K, V_hat) for the fp4 P.V workload."""
    vh = mx_dequantize_v(v_packed, v_scales, q.shape[2])
    return attention(q, k, vh, cu_seqlens_q, cu_seqlens_k, causal, softmax_scale, **kw)


def attention_fp4pv_sampled(q, k, v_packed, v_scales, cu_seqlens_q, cu_seqlens_k, causal: bool,
                            softmax_scale: float, samples):
    """Sampled-row version of ``attention_fp4pv``."""
    vh = mx_dequantize_v(v_packed, v_scales, q.shape[2])
    return attention_sampled(q, k, vh, cu_seqlens_q, cu_seqlens_k, causal, softmax_scale, samples)


def log2e_scale(softmax_scale: float) -> float:
    """c = tau * log2 e in fp64, tau = fp32(softmax_scale) (what the kernel receives)."""
    return float(np.float32(softmax_scale)) / float(np.log(2.0))


def group_exponents(raw_gmax: np.ndarray, c: float):
    """E_G = ceil(c g - log2 6) from the exact group maxima, in fp64.

    Returns (E as float64 with -inf for empty groups, the argument a = c g - log2 6).
    """
    with np.errstate(invalid="ignore"):
        arg = c * np.asarray(raw_gmax, dtype=np.float64) - LOG2_6
    return np.ceil(arg), arg


def _group_starts(key_tokens: np.ndarray):
    blk = np.asarray(key_tokens) // MX_BLOCK
    if not blk.size:
        return np.zeros(0, dtype=np.intp), np.zeros(0, dtype=np.intp)
    starts = np.flatnonzero(np.r_[True, blk[1:] != blk[:-1]])
    return starts, np.diff(np.r_[starts, blk.size])


def quantize_p_row_block(raw: np.ndarray, key_tokens: np.ndarray, c: float):
    """The P quantisation of rows of raw scores (masked keys = -inf).

    raw [r, sk] fp64 raw scores q.k of one (document, head); key_tokens [sk]
    the packed token index of each key (groups are the 32-token blocks).
    Returns (x [r, sk] = 2^(c r - E_G) before rounding, codes, E [r, sk]
    (each key's group exponent), and each key's group argument c g - log2 6).
    """
    starts, counts = _group_starts(key_tokens)
    gmax = (np.maximum.reduceat(raw, starts, axis=1) if starts.size
            else np.zeros((raw.shape[0], 0)))
    e_g, arg_g = group_exponents(gmax, c)
    e = np.repeat(e_g, counts, axis=1)
    arg = np.repeat(arg_g, counts, axis=1)
    finite = np.isfinite(raw)
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.where(finite, np.exp2(np.where(finite, c * raw - e, -np.inf)), 0.0)
    return x, e2m1_encode(x), e, arg


@dataclass
class FP4Emulation:
    out: np.ndarray        # [n, dv] emulated O
    lse: np.ndarray        # [n] LSE of the unquantised scores
    bound: np.ndarray      # [n, dv] bound on |O_emulated - O_exact|
    ambiguity: np.ndarray  # [n, dv] how far the fp32-ambiguous decisions can move O, in total
    group_tie: np.ndarray  # [n] bool: some group exponent is ambiguous
    key_tie: np.ndarray    # [n] int: keys whose e2m1 rounding is ambiguous
    # per row, the signed change of O that each ambiguous decision's other
    # branch makes ([K, dv], K = number of decisions), and what is left
    # unlisted (second-order: a rounding that is ambiguous only on the other
    # grid of an ambiguous group), as an elementwise allowance [dv]
    alternatives: list = None
    slack: np.ndarray = None


def _e2m1_neighbours(x: np.ndarray):
    """The e2m1 values just below and just above x (0 <= x <= 6)."""
    vals = e2m1_decode(_POS_CODES)
    hi_idx = np.clip(np.searchsorted(vals, x, side="left"), 1, 7)
    return vals[hi_idx - 1], vals[hi_idx]


def _fp4_rows(raw: np.ndarray, absdot: np.ndarray, key_tokens: np.ndarray, vh: np.ndarray,
              c: float, d: int):
    """Emulated O, LSE, error bound and ambiguity for rows of raw scores.

    absdot [r, sk] holds sum_t |q_t k_t| of each score (its fp32 error scale).
    """
    r, dv = raw.shape[0], vh.shape[1]
    if raw.shape[1] == 0:      # a document without keys: O = 0, LSE = -inf
        z = np.zeros((r, dv))
        return (z, np.full(r, -np.inf), z.copy(), z.copy(), np.zeros(r, dtype=bool),
                np.zeros(r, dtype=np.int64), [np.zeros((0, dv))] * r, z.copy())
    x, codes, e, arg = quantize_p_row_block(raw, key_tokens, c)
    finite = np.isfinite(raw)
    any_vis = finite.any(axis=1)
    with np.errstate(invalid="ignore"):
        m = np.where(any_vis, np.max(np.where(finite, c * raw, -np.inf), axis=1), 0.0)
        # everything relative to 2^m of the row: p_j = 2^(c r_j - m)
        p = np.where(finite, np.exp2(np.where(finite, c * raw, -np.inf) - m[:, None]), 0.0)
        rel = np.where(finite, np.exp2(np.where(finite, e, 0.0) - m[:, None]), 0.0)
    l = p.sum(axis=1)
    inv_l = np.where(any_vis, 1.0 / np.where(any_vis, l, 1.0), 0.0)
    p_hat = e2m1_decode(codes) * rel
    out = (p_hat @ vh) * inv_l[:, None]
    # |P_hat - p| <= 2^E * max(1/4, x/4): the e2m1 half-spacing below 2 is 1/4,
    # above 2 it is at most x/4
    err = rel * np.maximum(0.25, x / 4.0)
    bound = (err @ np.abs(vh)) * inv_l[:, None]

    # decision 1: a scaled value next to an e2m1 rounding midpoint; the other
    # branch takes the other neighbour of x on the grid
    raw0 = np.where(finite, raw, 0.0)
    x_err = fp32_window.rel_error_of_exp2(
        fp32_window.arg_error(c, raw0, absdot, d, np.where(finite, c * raw0 - e, 0.0)))
    key_amb = finite & fp32_window.within(_e2m1_midpoint_distance(x), x_err)
    lo, hi = _e2m1_neighbours(np.minimum(x, E2M1_MAX))
    chosen = e2m1_decode(codes)
    key_delta = np.where(key_amb, (np.where(chosen == hi, lo, hi) - chosen) * rel, 0.0)
    # decision 2: a group argument next to an integer. fp32 takes its maximum
    # over fp32 scores, so the argument is off by the largest score error in
    # the group; ceil may then land one lower or one higher, and the group's
    # keys follow that other grid
    starts, counts = _group_starts(key_tokens)
    sc_err = np.where(finite, fp32_window.score_error(absdot, d), 0.0)
    g_err = np.maximum.reduceat(sc_err, starts, axis=1)
    gmax = np.maximum.reduceat(raw, starts, axis=1)
    g_fin = np.isfinite(gmax)
    _, g_arg = group_exponents(np.where(g_fin, gmax, 0.0), c)
    a_err = np.where(g_fin, c * g_err + fp32_window.U32 * (c * np.abs(np.where(g_fin, gmax, 0.0))
                                                           + np.abs(g_arg) + 3.0), 0.0)
    win = fp32_window.SAFETY * a_err
    e_lo, e_hi = np.ceil(g_arg - win), np.ceil(g_arg + win)
    e_g = np.ceil(g_arg)
    g_alt = np.where(e_lo != e_g, e_lo, np.where(e_hi != e_g, e_hi, np.nan))
    g_tie = g_fin & np.isfinite(g_alt)
    tie = np.repeat(g_tie, counts, axis=1) & finite
    grp_delta = np.zeros_like(p_hat)
    alt_slack = np.zeros_like(p_hat)
    if tie.any():
        e_alt = np.repeat(np.where(g_tie, g_alt, 0.0), counts, axis=1)
        with np.errstate(invalid="ignore", over="ignore"):
            x_alt = np.where(tie, np.exp2(np.where(tie, c * raw - e_alt, -np.inf)), 0.0)
            rel_alt = np.where(tie, np.exp2(np.where(tie, e_alt, 0.0) - m[:, None]), 0.0)
        p_alt = e2m1_decode(e2m1_encode(x_alt)) * rel_alt
        grp_delta = np.where(tie, p_alt - p_hat, 0.0)
        alt_amb = tie & fp32_window.within(_e2m1_midpoint_distance(x_alt), x_err)
        alt_slack = np.where(alt_amb, rel_alt * _e2m1_step(x_alt), 0.0)
    ambiguity = ((np.abs(key_delta) + np.abs(grp_delta) + alt_slack) @ np.abs(vh)) * inv_l[:, None]
    slack = (alt_slack @ np.abs(vh)) * inv_l[:, None]
    # the signed effect of each decision on O, per row (ties are sparse)
    alternatives = []
    key_group = np.repeat(np.arange(starts.size), counts)
    for i in range(r):
        rows = []
        for j in np.flatnonzero(key_amb[i]):
            rows.append(key_delta[i, j] * vh[j] * inv_l[i])
        for gi in np.flatnonzero(g_tie[i]):
            members = np.flatnonzero(key_group == gi)
            rows.append((grp_delta[i, members] @ vh[members]) * inv_l[i])
        alternatives.append(np.array(rows).reshape(len(rows), dv))
    group_tie = tie.any(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, (m + np.log2(np.where(any_vis, l, 1.0))) * np.log(2.0), -np.inf)
    return (out, lse, bound, ambiguity, group_tie, key_amb.sum(axis=1), alternatives, slack)


def outcome_within(o: np.ndarray, out: np.ndarray, alternatives: np.ndarray, slack: np.ndarray,
                   bar: np.ndarray, max_enumerated: int = 10) -> bool:
    """Whether O of one row lies within ``bar`` (+ slack) of some outcome of the method.

    The outcomes are out + sum_k b_k alternatives[k] over b in {0, 1}^K: each
    ambiguous decision taken either way. With more than ``max_enumerated``
    decisions the largest are enumerated and the rest are added to the
    allowance by their magnitude.
    """
    alts = np.asarray(alternatives).reshape(-1, out.shape[-1])
    allow = bar + slack
    if alts.shape[0] > max_enumerated:
        order = np.argsort(-np.abs(alts).max(axis=1))
        allow = allow + np.abs(alts[order[max_enumerated:]]).sum(axis=0)
        alts = alts[order[:max_enumerated]]
    k = alts.shape[0]
    choices = ((np.arange(2 ** k)[:, None] >> np.arange(k)[None, :]) & 1).astype(np.float64)
    cands = out[None, :] + choices @ alts
    return bool((np.abs(o[None, :] - cands) <= allow[None, :]).all(axis=1).any())


def attention_fp4pv_emulated(q, k, v_packed, v_scales, cu_seqlens_q, cu_seqlens_k,
                             causal: bool, softmax_scale: float, samples=None) -> FP4Emulation:
    """The method's fp4 P.V result for (token, head) samples (all if None).

    ``samples`` is an iterable of (global query token, head); results follow its
    order. Each row is computed from its complete score row.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    total_q, h, dq = q.shape
    if samples is None:
        samples = [(t, hh) for t in range(total_q) for hh in range(h)]
    samples = list(samples)
    vh_all = mx_dequantize_v(v_packed, v_scales, dq)
    dv = vh_all.shape[2]
    c = log2e_scale(softmax_scale)
    n = len(samples)
    res = FP4Emulation(np.zeros((n, dv)), np.zeros(n), np.zeros((n, dv)), np.zeros((n, dv)),
                       np.zeros(n, dtype=bool), np.zeros(n, dtype=np.int64), [None] * n,
                       np.zeros((n, dv)))
    groups = {}
    for i, (t, hh) in enumerate(samples):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        groups.setdefault((b, int(hh)), []).append((i, int(t)))
    for (b, hh), items in groups.items():
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        kb = _as_f64(k[k0:k1, hh, :])
        vb = vh_all[k0:k1, hh, :]
        key_tokens = np.arange(k0, k1)
        for s0 in range(0, len(items), 512):
            part = items[s0:s0 + 512]
            idx = np.array([t for _, t in part])
            qb = _as_f64(q[idx.tolist(), hh, :])
            raw = qb @ kb.T
            absdot = np.abs(qb) @ np.abs(kb).T
            vis = visible(idx - q0, q1 - q0, k1 - k0, causal)
            raw = np.where(vis, raw, -np.inf)
            o, lse, bound, amb, tie, nk, alts, slack = _fp4_rows(raw, absdot, key_tokens, vb, c,
                                                                 dq)
            rows = np.array([i for i, _ in part])
            res.out[rows], res.lse[rows], res.bound[rows] = o, lse, bound
            res.ambiguity[rows], res.group_tie[rows], res.key_tie[rows] = amb, tie, nk
            res.slack[rows] = slack
            for i_row, a in zip(rows, alts):
                res.alternatives[i_row] = a
    return res


def attention_fp4pv_bruteforce(q, k, v_packed, v_scales, cu_seqlens_q, cu_seqlens_k,
                               causal: bool, softmax_scale: float):
    """Pure-Python loops over rows, groups and keys; tiny inputs only.

    Same quantisation as ``attention_fp4pv_emulated`` written element by
    element (group scale from the group's largest score, nearest e2m1 by
    search over the grid, ties to the even code), so that it can pin the
    vectorised version. Returns O [total_q, h, dv].
    """
    import math
    qf, kf = _as_f64(q), _as_f64(k)
    vh = mx_dequantize_v(v_packed, v_scales, qf.shape[2])
    c = log2e_scale(softmax_scale)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    total_q, h, d = qf.shape
    dv = vh.shape[2]
    out = np.zeros((total_q, h, dv))

    def nearest(xv):
        xv = min(xv, 6.0)
        best = min(range(8), key=lambda i: (abs(grid[i] - xv), i % 2))
        return grid[best]

    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        for hh in range(h):
            for i in range(sq):
                vis = [j for j in range(sk) if (not causal) or j <= i + sk - sq]
                if not vis:
                    continue
                raw = {j: math.fsum(float(qf[q0 + i, hh, t]) * float(kf[k0 + j, hh, t])
                                    for t in range(d)) for j in vis}
                top = max(c * r for r in raw.values())
                weights = {}
                for blk in sorted({(k0 + j) // MX_BLOCK for j in vis}):
                    members = [j for j in vis if (k0 + j) // MX_BLOCK == blk]
                    g = max(raw[j] for j in members)
                    eg = math.ceil(c * g - math.log2(6.0))
                    for j in members:
                        weights[j] = nearest(2.0 ** (c * raw[j] - eg)) * 2.0 ** (eg - top)
                lsum = math.fsum(2.0 ** (c * raw[j] - top) for j in vis)
                for t in range(dv):
                    out[q0 + i, hh, t] = math.fsum(weights[j] * vh[k0 + j, hh, t] for j in vis) / lsum
    return out
