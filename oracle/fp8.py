"""OCP FP8 E4M3 decoding/encoding and the fp8 P.V oracle.

TEST INFRASTRUCTURE (see ``oracle/reference.py``): imported only by tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py``.

The fp8 P.V variant ("Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
GB300)", introduction and section 5) runs the second GEMM with P and V in
e4m3. V reaches the kernel as e4m3 codes plus one fp32 scale per head. The
oracle's answer for that workload is the exact attention of the inputs the
kernel receives: Q and K in bf16 and V_hat = decode(codes) * scale[h], all in
fp64. Rounding P to e4m3 is the kernel's approximation and is judged by the
looser fp8 tolerance.

E4M3 (OCP 8-bit floating point, "FN" variant): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the
codes S.1111.111 are NaN and there is no infinity; the largest finite value is
1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np

from .reference import attention, attention_sampled

E4M3_MAX = 448.0


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


def attention_fp8pv_emulated(q, k, v_codes, v_scale, cu_seqlens_q, cu_seqlens_k, causal: bool,
                             softmax_scale: float, p_scale_log2: float = 8.0):
    """Diagnostic CPU emulation of the P quantisation (not a parity reference).

    Per row, with m the row maximum of the scaled scores in base-2 units,
    P_hat = e4m3(2^(s*log2e - m + p_scale_log2)); O = scale[h] * sum P_hat V_codes /
    (2^p_scale_log2 * sum 2^(s*log2e - m)). The power-of-two P scale sits inside
    the exponent, as the log-domain refactoring of "Kernel Bottleneck Tuning",
    section 4, does with multiplicative scales. The GPU kernel quantises against
    a running maximum instead of the final one, so the two agree only within the
    fp8 tolerance, not bitwise.
    """
    from .reference import _as_f64, visible
    qf, kf = _as_f64(q), _as_f64(k)
    codes = v_codes.numpy() if hasattr(v_codes, "numpy") else np.asarray(v_codes)
    vq = e4m3_decode(codes)
    scale = v_scale.double().numpy() if hasattr(v_scale, "double") else np.asarray(v_scale, np.float64)
    tau = float(np.float32(softmax_scale))
    total_q, h, _ = qf.shape
    dv = vq.shape[2]
    out = np.zeros((total_q, h, dv))
    lse = np.full((h, total_q), -np.inf)
    log2e = 1.0 / np.log(2.0)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        for hh in range(h):
            s2 = tau * log2e * (qf[q0:q1, hh] @ kf[k0:k1, hh].T)
            vis = visible(np.arange(sq), sq, sk, causal)
            s2 = np.where(vis, s2, -np.inf)
            m = s2.max(axis=1) if sk else np.full(sq, -np.inf)
            ok = np.isfinite(m)
            m0 = np.where(ok, m, 0.0)
            e = np.exp2(s2 - m0[:, None])
            l = e.sum(axis=1)
            ph = e4m3_decode(e4m3_encode(np.minimum(e * 2.0 ** p_scale_log2, E4M3_MAX)))
            num = ph @ vq[k0:k1, hh]
            den = np.where(ok, l * 2.0 ** p_scale_log2, 1.0)
            out[q0:q1, hh] = np.where(ok[:, None], scale[hh] * num / den[:, None], 0.0)
            with np.errstate(divide="ignore"):
                lse[hh, q0:q1] = np.where(ok, (m0 + np.log2(np.where(ok, l, 1.0))) * np.log(2.0), -np.inf)
    return out, lse
