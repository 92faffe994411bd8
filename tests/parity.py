"""Comparison helpers shared by the parity tests (test infrastructure).

The stated bars ("O within atol + rtol |O_ref| elementwise, LSE within
1e-3") are checked by the tests themselves; this module holds the checks that
several test files use, and the error summary the tests report: the maximum
absolute error, the maximum error normalised by the row RMS of O_ref (so that
a wrong output stays visible on long rows, where |O_ref| is about 0.01 and an
absolute tolerance is loose), the RMS error, the count of elements over the
bar and the worst location.
"""

from __future__ import annotations

import numpy as np

# A kernel's O against the fp64 oracle differs by the rounding of P to bf16
# before P.V (relative 2^-9 per term, independent across keys) and of O to
# bf16 (relative 2^-9): per row, a few times 2^-9 of the row's RMS. The
# derived bar on the normalised error is 0.05 (about 25 times 2^-9), far
# below what a wrong output reaches (an all-zero row: max|O| / RMS(O), 2 to 3).
NORMALISED_BAR = 0.05


def error_summary(o: np.ndarray, o_ref: np.ndarray, atol: float, rtol: float,
                  extra: np.ndarray = None) -> dict:
    """Errors of o [n, d] against o_ref [n, d] (rows with O_ref = 0 excluded
    from the normalised error)."""
    o = np.asarray(o, np.float64).reshape(-1, o_ref.shape[-1])
    o_ref = np.asarray(o_ref, np.float64).reshape(-1, o.shape[-1])
    err = np.abs(o - o_ref)
    tol = atol + rtol * np.abs(o_ref)
    if extra is not None:
        tol = tol + extra.reshape(tol.shape)
    bad = err > tol
    rms = np.sqrt((o_ref ** 2).mean(axis=1))
    live = rms > 0
    norm = np.zeros(o.shape[0])
    norm[live] = err[live].max(axis=1) / rms[live]
    worst = np.unravel_index(int(np.argmax(err - tol)), err.shape)
    return {
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_normalised_err": float(norm.max()) if norm.size else 0.0,
        "worst_normalised_row": int(np.argmax(norm)) if norm.size else -1,
        "rms_err": float(np.sqrt((err ** 2).mean())) if err.size else 0.0,
        "n_over_bar": int(bad.sum()),
        "worst_location": tuple(int(i) for i in worst),
        "normalised_per_row": norm,
    }


def fp8_emulation_check(o: np.ndarray, emu) -> np.ndarray:
    """Per row: O within the bf16 bar of the emulated fp8 method, widened only
    by the oracle's fp32 ambiguity and subnormal-band allowances."""
    bar = 1e-2 + 1e-2 * np.abs(emu.out) + emu.ambiguity + emu.slack
    return np.all(np.abs(np.asarray(o) - emu.out) <= bar, axis=1)
