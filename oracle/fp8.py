"""OCP FP8 E4M3 decoding/encoding and the fp8 P.V oracle.

TEST INFRASTRUCTURE (see ``oracle/reference.py``): imported only by tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py``.

The fp8 P.V variant ("Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
GB300)", introduction and section 5) runs the second GEMM with P and V in
e4m3. V reaches the kernel as e4m3 codes plus one fp32 scale per head. Two
answers are computed:

  * ``attention_fp8pv``: the exact attention of the inputs the kernel
    receives, Q and K in bf16 and V_hat = decode(codes) * scale[h], in fp64;
    rounding P to e4m3 is the method's approximation, judged by the looser
    fp8 tolerance;
  * ``attention_fp8pv_emulated``: the method's quantised result. With
    c = tau log2 e and z_j = 2^(c s_j) the unnormalised exp2 weight of key j,
    the method rounds P in the log domain ("Kernel Bottleneck Tuning", section
    4: the scale is an addend of the exp2 argument) as
        P_hat_j = 2^(A - 5) e4m3(2^(c s_j - A + 5))
    with the anchor A = a + K: a = c m0, m0 the row's largest score among the
    document's first 64 keys (the first tile, where the row's first maximum
    is taken), and K a whole number of steps. Scaling by a power of two
    commutes with rounding to e4m3 while the value stays in its normal range,
    so P_hat_j = 2^a R(z_j / 2^a), with R the rounding to e4m3 precision (4
    significant bits, to nearest, ties to even), whatever K is; the first
    tile's largest key maps exactly. The row sum keeps the unquantised z, so
        O = scale[h] sum_j P_hat_j codes_j / sum_j z_j,  LSE = ln sum_j exp(tau s_j).
    Keys more than 2^11 below the anchor can fall in e4m3's subnormal range,
    where the rounding depends on K: the oracle takes K at its largest
    possible value and allows, per such key, what a smaller K can change
    (``slack``). Where fp32 scores may round a weight the other way (it sits
    next to an e4m3 midpoint closer than ``oracle.fp32_window`` trusts fp32,
    anchor included), the other rounding's effect on O is summed into
    ``ambiguity``.

E4M3 (OCP 8-bit floating point, "FN" variant): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the
codes S.1111.111 are NaN and there is no infinity; the largest finite value is
1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np

from dataclasses import dataclass

from . import fp32_window
from .reference import _as_f64, attention, attention_sampled, visible

E4M3_MAX = 448.0
P_SCALE_LOG2 = 5              # the method's P scale, 2^5, an addend of the exp2 argument
E4M3_MIN_NORMAL_LOG2 = -6     # smallest normal e4m3 value 2^-6
E4M3_SUBNORMAL_STEP_LOG2 = -9  # spacing of the subnormal e4m3 values
FIRST_TILE_KEYS = 64           # keys of the tile where a row's first maximum is taken


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 e4m3 codes to float64 from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


def _all_finite_values() -> tuple:
    codes = np.arange(128, dtype=np.uint8)          # non-negative half
    vals = e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values to the nearest e4m3 code, ties to an even code.

    Magnitudes above 448 saturate to 448 (the callers clamp first anyway);
    NaN maps to the NaN code 0x7F. The result is chosen by exhaustive search
    over the 127 finite non-negative codes, which is slow but plainly correct.
    """
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _all_finite_values()
    a = np.minimum(np.abs(x), E4M3_MAX)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    # distances to every candidate; pick the nearest, ties to even mantissa code
    chunk = 1 << 16
    for s in range(0, flat.size, chunk):
        seg = flat[s:s + chunk]
        d = np.abs(seg[:, None] - vals[None, :])
        best = d.min(axis=1, keepdims=True)
        tie = d == best
        # among ties prefer the even code
        even = (codes[None, :] & 1) == 0
        pick = np.where((tie & even).any(axis=1), np.argmax(tie & even, axis=1), np.argmax(tie, axis=1))
        out[s:s + chunk] = codes[pick]
    out = out.reshape(a.shape)
    neg = np.signbit(x) & (out != 0)
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out).astype(np.uint8)


def dequantize_v(v_codes, v_scale) -> np.ndarray:
    """V_hat[t, h, :] = decode(codes[t, h, :]) * scale[h] in fp64."""
    codes = v_codes.numpy() if hasattr(v_codes, "numpy") else np.asarray(v_codes)
    scale = v_scale.double().numpy() if hasattr(v_scale, "double") else np.asarray(v_scale, np.float64)
    return e4m3_decode(codes) * scale[None, :, None]


def attention_fp8pv(q, k, v_codes, v_scale, cu_seqlens_q, cu_seqlens_k, causal: bool,
                    softmax_scale: float, **kw):
    """Exact attention of (Q, K, V_hat) for the fp8 P.V workload."""
    return attention(q, k, dequantize_v(v_codes, v_scale), cu_seqlens_q, cu_seqlens_k, causal,
                     softmax_scale, **kw)


def attention_fp8pv_sampled(q, k, v_codes, v_scale, cu_seqlens_q, cu_seqlens_k, causal: bool,
                            softmax_scale: float, samples):
    """Sampled-row version of ``attention_fp8pv``."""
    return attention_sampled(q, k, dequantize_v(v_codes, v_scale), cu_seqlens_q, cu_seqlens_k,
                             causal, softmax_scale, samples)


def round_e4m3(x) -> np.ndarray:
    """Round non-negative float64 values to the nearest e4m3 value, ties to even.

    Written from the format: a normal value keeps 4 significant bits, so
    x = f 2^e with f in [0.5, 1) rounds to rint(16 f) 2^(e - 4) (numpy's rint
    rounds halves to even, which is the even mantissa code); below 2^-6 the
    values are multiples of 2^-9. Magnitudes above 448 saturate. The
    exhaustive ``e4m3_encode`` pins it (tests/test_oracle_fp8.py).
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    normal = np.ldexp(np.rint(16.0 * f), e - 4)
    sub = np.ldexp(np.rint(np.ldexp(x, 9)), -9)
    return np.minimum(np.where(x < 2.0 ** E4M3_MIN_NORMAL_LOG2, sub, normal), E4M3_MAX)


def _e4m3_midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Relative distance of x (> 0, e4m3 range) to the nearest e4m3 rounding midpoint."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    step = np.where(x < 2.0 ** E4M3_MIN_NORMAL_LOG2, 2.0 ** E4M3_SUBNORMAL_STEP_LOG2,
                    np.ldexp(1.0, e - 4))
    t = x / step
    d = np.abs(t - (np.floor(t) + 0.5)) * step
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(x > 0, d / x, np.inf)


def _e4m3_step(x: np.ndarray) -> np.ndarray:
    """Spacing of the e4m3 values around x (the cost of a flipped rounding)."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.where(x < 2.0 ** E4M3_MIN_NORMAL_LOG2, 2.0 ** E4M3_SUBNORMAL_STEP_LOG2,
                    np.ldexp(1.0, e - 4))


@dataclass
class FP8Emulation:
    out: np.ndarray        # [n, dv] emulated O
    lse: np.ndarray        # [n] LSE of the unquantised scores
    bound: np.ndarray      # [n, dv] |O_emulated - O_exact| bound (sum |R(z) - z| |V| / l)
    ambiguity: np.ndarray  # [n, dv] how far fp32-ambiguous roundings can move O, in total
    slack: np.ndarray      # [n, dv] what the subnormal band's dependence on M can change
    key_tie: np.ndarray    # [n] int: keys whose rounding is ambiguous


def log2e_scale(softmax_scale: float) -> float:
    """c = tau * log2 e in fp64, tau = fp32(softmax_scale) (what the kernel receives)."""
    return float(np.float32(softmax_scale)) / float(np.log(2.0))


def _fp8_rows(raw: np.ndarray, absdot: np.ndarray, vq: np.ndarray, c: float, d: int):
    """Emulated O (before the per-head V scale), LSE, bound, ambiguity, slack.

    raw [r, sk] holds the rows' raw scores over the document's keys in order
    (masked keys -inf); absdot the sums of |q_t k_t| (fp32 error scales)."""
    r, dv = raw.shape[0], vq.shape[1]
    finite = np.isfinite(raw)
    any_vis = finite.any(axis=1)
    raw0 = np.where(finite, raw, 0.0)
    with np.errstate(invalid="ignore"):
        top = np.where(any_vis, np.max(np.where(finite, c * raw, -np.inf), axis=1), 0.0)
        first = raw[:, :FIRST_TILE_KEYS]
        first_vis = np.isfinite(first).any(axis=1)
        a = np.where(first_vis, c * np.max(np.where(np.isfinite(first), first, -np.inf), axis=1),
                     top)
    sc_err = fp32_window.score_error(absdot, d)
    # fp32 forms the first anchor from the largest fp32 score of the first tile
    a_err = np.where(any_vis, c * np.max(np.where(np.isfinite(first),
                                                  sc_err[:, :FIRST_TILE_KEYS], 0.0), axis=1),
                     0.0) + 3 * fp32_window.U32 * np.abs(a)
    top_err = np.where(any_vis, np.max(np.where(
        finite, fp32_window.arg_error(c, raw0, absdot, d, c * raw0), 0.0), axis=1), 0.0)
    # the highest anchor the row can reach: a plus the whole steps to the row's
    # largest weight, with fp32's error taken in the direction of more steps
    k_hi = np.maximum(np.ceil(top - a + fp32_window.SAFETY * (top_err + a_err)), 0.0)
    a_hi = a + k_hi
    # x = 2^(c s - A + 5) at A = a_hi; weights z relative to 2^a_hi
    with np.errstate(invalid="ignore", over="ignore"):
        arg = np.where(finite, c * raw0 - a_hi[:, None] + P_SCALE_LOG2, -np.inf)
        x = np.where(finite, np.exp2(arg), 0.0)
    xq = round_e4m3(x)
    scale_row = 2.0 ** -P_SCALE_LOG2
    z = x * scale_row
    ref = xq * scale_row
    l = z.sum(axis=1)
    inv_l = np.where(any_vis, 1.0 / np.where(any_vis, l, 1.0), 0.0)
    out = (ref @ vq) * inv_l[:, None]
    bound = (np.abs(ref - z) @ np.abs(vq)) * inv_l[:, None]
    # keys normal at every anchor the row can reach: x >= 2^-6 at the highest
    tail = finite & (x < 2.0 ** E4M3_MIN_NORMAL_LOG2)
    # a tail key rounds within min(z, half a subnormal step at a_hi) + 2^-4 z of z
    # whatever the steps are, and so does the reference: twice that between them
    half_sub = 2.0 ** (E4M3_SUBNORMAL_STEP_LOG2 - 1) * scale_row
    tail_gap = np.where(tail, 2.0 * (np.minimum(z, half_sub) + z / 16.0), 0.0)
    slack = (tail_gap @ np.abs(vq)) * inv_l[:, None]
    # normal-range keys next to a rounding midpoint: the argument's fp32 error
    # is its own plus the anchor's (first anchor, whole steps added in fp32,
    # and the addend 5 - A)
    anchor_err = a_err + fp32_window.U32 * (2 * np.abs(a_hi) + P_SCALE_LOG2)
    x_err = fp32_window.rel_error_of_exp2(
        fp32_window.arg_error(c, raw0, absdot, d, np.where(finite, arg, 0.0))
        + anchor_err[:, None])
    amb_key = finite & ~tail & fp32_window.within(_e4m3_midpoint_distance(x), x_err)
    amb = np.where(amb_key, _e4m3_step(x) * scale_row, 0.0)
    ambiguity = (amb @ np.abs(vq)) * inv_l[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, (a_hi + np.log2(np.where(any_vis, l, 1.0))) * np.log(2.0),
                       -np.inf)
    return out, lse, bound, ambiguity, slack, amb_key.sum(axis=1)


def attention_fp8pv_emulated(q, k, v_codes, v_scale, cu_seqlens_q, cu_seqlens_k, causal: bool,
                             softmax_scale: float, samples=None) -> FP8Emulation:
    """The method's fp8 P.V result for (token, head) samples (all if None).

    ``samples`` is an iterable of (global query token, head); results follow
    its order, each row computed from its complete score row.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    total_q, h, dq = q.shape
    if samples is None:
        samples = [(t, hh) for t in range(total_q) for hh in range(h)]
    samples = list(samples)
    codes = v_codes.numpy() if hasattr(v_codes, "numpy") else np.asarray(v_codes)
    vq_all = e4m3_decode(codes)
    vs = (v_scale.double().numpy() if hasattr(v_scale, "double")
          else np.asarray(v_scale, np.float64))
    dv = vq_all.shape[2]
    c = log2e_scale(softmax_scale)
    n = len(samples)
    res = FP8Emulation(np.zeros((n, dv)), np.zeros(n), np.zeros((n, dv)), np.zeros((n, dv)),
                       np.zeros((n, dv)), np.zeros(n, dtype=np.int64))
    groups = {}
    for i, (t, hh) in enumerate(samples):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        groups.setdefault((b, int(hh)), []).append((i, int(t)))
    for (b, hh), items in groups.items():
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        kb = _as_f64(k[k0:k1, hh, :])
        vb = vq_all[k0:k1, hh, :]
        for s0 in range(0, len(items), 256):
            part = items[s0:s0 + 256]
            idx = np.array([t for _, t in part])
            rows = np.array([i for i, _ in part])
            if k1 == k0:       # a document without keys: O = 0, LSE = -inf
                res.lse[rows] = -np.inf
                continue
            qb = _as_f64(q[idx.tolist(), hh, :])
            raw = qb @ kb.T
            absdot = np.abs(qb) @ np.abs(kb).T
            vis = visible(idx - q0, q1 - q0, k1 - k0, causal)
            raw = np.where(vis, raw, -np.inf)
            o, lse, bound, amb, slack, nk = _fp8_rows(raw, absdot, vb, c, dq)
            sv = vs[hh]
            res.out[rows], res.lse[rows], res.bound[rows] = sv * o, lse, sv * bound
            res.ambiguity[rows], res.slack[rows], res.key_tie[rows] = sv * amb, sv * slack, nk
    return res


def attention_fp8pv_bruteforce(q, k, v_codes, v_scale, cu_seqlens_q, cu_seqlens_k,
                               causal: bool, softmax_scale: float):
    """Pure-Python loops over rows and keys; tiny inputs only.

    The method's weights written element by element from the definition: with
    a = c m0 (m0 the row's largest visible score among the document's first 64
    keys), each w_j = 2^(c s_j - a) rounded to the nearest value with 4
    significant bits (the candidates (8 + i) 2^(e - 3), i = 0..8, around
    2^e <= w_j < 2^(e+1); ties to an even i), O = scale[h] sum R(w_j) V_j /
    sum w_j. For inputs whose weights all lie within 2^11 of the anchor (no
    subnormal band). Returns O [total_q, h, dv].
    """
    import math
    qf, kf = _as_f64(q), _as_f64(k)
    codes = v_codes.numpy() if hasattr(v_codes, "numpy") else np.asarray(v_codes)
    vq = e4m3_decode(codes)
    vs = (v_scale.double().numpy() if hasattr(v_scale, "double")
          else np.asarray(v_scale, np.float64))
    c = float(np.float32(softmax_scale)) / math.log(2.0)
    total_q, h, d = qf.shape
    dv = vq.shape[2]
    out = np.zeros((total_q, h, dv))

    def r4(wv):
        e = math.floor(math.log2(wv))
        cands = [(8 + i) * 2.0 ** (e - 3) for i in range(9)]
        return cands[min(range(9), key=lambda i: (abs(cands[i] - wv), i % 2))]

    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        for hh in range(h):
            for i in range(sq):
                vis = [j for j in range(sk) if (not causal) or j <= i + sk - sq]
                if not vis:
                    continue
                s = {j: math.fsum(float(qf[q0 + i, hh, t]) * float(kf[k0 + j, hh, t])
                                  for t in range(d)) for j in vis}
                a = c * max(s[j] for j in vis if j < FIRST_TILE_KEYS)
                w = {j: 2.0 ** (c * s[j] - a) for j in vis}
                lsum = math.fsum(w.values())
                for t in range(dv):
                    out[q0 + i, hh, t] = vs[hh] * math.fsum(r4(w[j]) * vq[k0 + j, hh, t]
                                                            for j in vis) / lsum
    return out
